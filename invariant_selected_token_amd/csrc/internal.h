// internal.h -- launch interface between the C ABI layer (api.hip) and the
// kernels (kernels.hip).  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rlk {

// Workgroup tile of the logit GEMM: TILE_V vocabulary rows x TILE_T token
// rows, the full hidden dimension per workgroup, the same for every batch
// size.  Each wave covers 128 x 128 of it; STAT_V = 128 is the width of the
// vocabulary tiles whose (max, sum of exponentials) statistics are merged, so
// it is part of the numerical contract.
constexpr int TILE_V = 256;
constexpr int STAT_V = 128;
constexpr int TILE_T = 256;
constexpr int TILE_K = 64;
constexpr int GEMM_THREADS = 256;
// The vocabulary merge: MERGE_GROUPS contiguous groups of vocabulary tiles
// per row (part of the numerical contract), MERGE_ROWS rows per workgroup;
// groups of up to MERGE_KEEP tiles are held in registers.
constexpr int MERGE_GROUPS = 16;
constexpr int MERGE_ROWS = 32;
constexpr int MERGE_KEEP = 80;
constexpr int MERGE_UNROLL = 16;
constexpr int COMPARE_THREADS = 1024;
constexpr int COMPARE_UNROLL = 4;

struct GemmArgs {
  const uint16_t *hidden;
  const uint16_t *weight;
  const int32_t *targets;
  float *part_m;   // [nST][T] per-statistics-tile maxima
  float *part_s;   // [nST][T] per-statistics-tile sums of exp(z - m)
  float *xt;       // [T] target logits
  float *logits;   // [T][V] (logits stage only)
  float *part_u;   // [nST][T] per-tile sums of exp(z - m) (z - m) (entropy only)
  // Contract options (statistics kernel, ex variants only): every logit is
  // multiplied by inv_tau and, when bf16_logits, rounded to bf16.
  float inv_tau;
  int bf16_logits;
  // 0: plain statistics; 1: with the options; 2: options and entropy partials;
  // 3: the backward's logit gradient instead of statistics
  int ex;
  int pf_hidden;  // plain GEMM: also prefetch the hidden-role operand into L2
  // 8 per-XCD tile-claim counters (zeroed by the launcher before the kernel),
  // or null for the fixed walk
  int *queue;
  // Logit gradient (ex == 3): dz = g inv_tau (onehot(y) - exp(z inv_tau - lse))
  // rounded to bf16, written to dz [T][ld_dz] (columns V .. Vp-1 zero).
  const float *lse;
  const float *grad;
  uint16_t *dz;
  int64_t ld_dz;
  int Vp;
  // Plain GEMM: the weight-role operand stored K-major, [depth][kcols
  // columns] with the depth along its rows (the product over the vocabulary
  // reads the weight as it is stored); kr is its number of rows along the
  // depth (rows kr .. H-1 of the depth read as zeros); kcols >= V columns
  // are read (a multiple of 8; columns V .. kcols-1 reach only outputs that
  // are not stored).
  int kmw;
  int kr;
  int kcols;
  // Plain GEMM: store the output transposed, out[v][t] with row stride T
  // (logits then points at a [V][T] fp32 array).  K-major weight role only.
  int out_t;
  int64_t ldh;
  int64_t ldw;
  int T;
  int H;
  int V;
  int js_base;  // global index of this weight slice's first statistics tile
  int y_base;   // global vocabulary index of this weight slice's first row
  int nMT;   // token tiles, ceil(T / TILE_T)
  int nVT;   // workgroup vocabulary tiles, ceil(V / TILE_V)
  int nST;   // statistics tiles, ceil(V / STAT_V)
};

struct MergeArgs {
  const float *part_m;
  const float *part_s;
  const float *xt;
  const float *part_u;   // entropy partials (when entropy != nullptr)
  const int32_t *targets;
  float *logp;
  float *lse;
  float *entropy;        // nullptr: no entropy
  int T;
  int V;
  int nST;
};

inline int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// `workers`: workgroups of the persistent statistics kernel (the device's
// compute-unit count); it changes the schedule, never the results.
hipError_t launch_gemm_stats(const GemmArgs &a, int workers, hipStream_t s);
hipError_t launch_gemm_logits(const GemmArgs &a, int workers, hipStream_t s);
hipError_t launch_merge(const MergeArgs &a, hipStream_t s);
// out[c][r] = in[r][c] for r < R, c < C, and 0 for R <= r < ldo (bf16 bits);
// C % 64 == 0, ldi % 8 == 0, ldo % 64 == 0, 16-byte aligned pointers.
hipError_t launch_transpose(const uint16_t *in, int64_t ldi, int R, int C, uint16_t *out,
                            int64_t ldo, hipStream_t s);
// RMSNorm of T rows (bf16 [T][ldx]) with weight gamma (bf16 [H]) into y; H % 8
// == 0, ldx and ldy multiples of 8, 16-byte aligned pointers.
hipError_t launch_rmsnorm(const uint16_t *x, int64_t ldx, const uint16_t *gamma, float eps,
                          uint16_t *y, int64_t ldy, int T, int H, hipStream_t s);
// Top-k log-probabilities of T rows of stored fp32 logits [T][ld] (1 <= k <= 64),
// filtered by the statistics pass's tile maxima part_m [ceil(V/128)][T].
hipError_t launch_topk(const float *logits, int64_t ld, const float *lse, const float *part_m,
                       int T, int V, int k, float inv_tau, int bf16, float *out_lp,
                       int32_t *out_id, hipStream_t s);
// Top-k log-probabilities without stored logits: the candidate tiles of
// every row (from the statistics pass's tile maxima) are recomputed by the
// logit GEMM's MFMA chain into pair_z, 128 raw logits per (row, tile) pair,
// and the selection reads them there.  Buffers are carved from the caller's
// workspace (see rlk_topk_logp_direct); C = k pair slots per row, then
// dcap * nST pairs for rows whose k-th largest tile maximum is -inf when
// nST > C.
struct TopkDirectArgs {
  const uint16_t *hidden;
  const uint16_t *weight;
  int64_t ldh;
  int64_t ldw;
  const float *lse;
  const float *part_m;   // [nST][T], the statistics pass's tile maxima
  float *out_lp;
  int32_t *out_id;
  float *pair_z;         // [P][128]
  int *bucket;           // [P] pair ids grouped by tile
  int *cand_tile;        // [T][C]
  int *cand_n;           // [T]
  int *deg_rank;         // [T]
  int *deg_row;          // [max(dcap, 1)]
  int *tile_count;       // [nST]
  int *tile_off;         // [nST]
  int *tile_fill;        // [nST]
  int *item_off;         // [nST + 1]
  int *item_tile;        // [items_max]
  int *totals;           // [2]: work items, pairs
  float inv_tau;
  int bf16;
  int T, H, V, nST, k, C, dcap;
  int tl_pairs;   // pairs per work item of the tile logits: 128 (4 waves), 256 (8 waves)
  int items_max;
};
hipError_t launch_topk_direct(const TopkDirectArgs &a, hipStream_t s);
// x[0 .. n) = 0.0f
hipError_t launch_zero(float *x, int64_t n, hipStream_t s);
hipError_t launch_compare(const float *a, const float *b, int64_t n,
                          double *stats, hipStream_t s);

}  // namespace rlk
