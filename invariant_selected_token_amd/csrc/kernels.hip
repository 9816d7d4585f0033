// kernels.hip -- gfx950 kernels of the batch-invariant selected-token
// log-probability path.
//
//   gemm_kernel<true,.> logits z = W . h^T on bf16 MFMA with fp32 accumulation
//                       (RL-Kernel blog, section 二: the K split of a GEMM is a
//                       source of drift; sections 六/七: one workgroup per
//                       output tile, full K in a fixed order, no split-K),
//                       with the per-(row, vocabulary tile) max and sum of
//                       exponentials and the target-logit capture fused into
//                       its epilogue (section 四: per-block m_j, s_j of the
//                       LSE; section 七: local statistics per vocabulary
//                       tile, here 128 wide).  Logits never leave registers.
//   gemm_kernel<false,.> the same main loop, storing fp32 logits (the
//                       stage-by-stage comparison of section 五; also the two
//                       gradient products of the backward).  EX 0 stores 16
//                       bytes per lane, EX 1 one column per store, for rows
//                       whose length or base is not 16-byte aligned, EX 2
//                       each tile transposed (out[v][t]).  KMW reads the
//                       weight-role operand K-major (stored with the depth
//                       along its rows) through the transposing LDS read:
//                       the product over the vocabulary takes the weight,
//                       and the product over the tokens takes dz, as they
//                       are stored.
//   merge_kernel        per row, folds the tile statistics in a fixed order
//                       that depends only on the number of vocabulary tiles,
//                       then lse = M + log(s) and logp = z_y - lse (and, with
//                       the entropy partials, H = log S - U / S).
//
// Contract options (the EX instantiations of the statistics kernel): the
// logits are multiplied by 1/tau (sampling temperature) and optionally
// rounded to bf16 (engines that keep a bf16 logits tensor; the blog's
// sections 二/四 name that cast as a drift point) before the statistics and
// the target capture; with EX == 2 each tile also yields
// u = sum exp(z - m) (z - m), from which the merge forms the entropy.
//   rmsnorm_kernel      the RMSNorm feeding the LM head, one wave per row with
//                       a fixed reduction order over the hidden dimension
//                       (section 四 lists RMSNorm among the reductions whose
//                       order matters).
//   topk_kernel         the k largest log-probabilities of a row from stored
//                       logits (same options, same subtraction as the merge).
//   topk_cand_*, topk_plan_kernel, topk_scatter_kernel, tile_logits_kernel,
//   topk_select_wave_kernel
//                       the same top-k without stored logits: each row's
//                       candidate tiles, bucketed by tile, recomputed by the
//                       logit GEMM's MFMA chain, then selected.
//   transpose_kernel    h^T for the backward's product over the tokens
//                       (64 x 64 tiles through LDS).
//   compare_kernel      mismatch count / max |diff| / k3 of two fp32 arrays
//                       (sections 六/七; the vLLM blog summary's diff = 0).
//
// Why rows are batch invariant: every output z[t][v] is produced by the same
// chain of MFMA instructions over k in increasing order whatever tile or tile
// position row t lands in; one 256 x 256 tile serves every batch size, and
// rows past T only change which loads are issued (their accumulators are
// never written); vocabulary rows beyond V read as zeros through the buffer
// unit's range check; the epilogue's reduction tree for a row depends only on
// the tile geometry; the merge's fold depends only on ceil(V / STAT_V).  No
// split-K.  The one atomic operation, a workgroup claiming its next tile from
// a counter, only decides which workgroup computes a tile, never what it
// computes.
#include <hip/hip_runtime.h>
#include <float.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "internal.h"

namespace rlk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int STAGE_BYTES = TILE_V * TILE_K * 2;  // one operand, one stage
constexpr int GROUP_M = 4;   // token tiles that walk the vocabulary together
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
// Buffer resource word 3 for gfx9-family raw buffers (32-bit data format).
constexpr int RSRC_WORD3 = 0x00020000;
// s_waitcnt immediate for "vmcnt(0)" only (expcnt and lgkmcnt left at their
// maxima).
constexpr int VMCNT0 = 0x0F70;
// "vmcnt(1) lgkmcnt(0)", "vmcnt(2) lgkmcnt(0)" and "vmcnt(0) lgkmcnt(0)"
constexpr int VMCNT1_LGKMCNT0 = 0x0071;
constexpr int VMCNT2_LGKMCNT0 = 0x0072;
constexpr int VMCNT0_LGKMCNT0 = 0x0070;
// K blocks between an L2 prefetch of weight rows and the block's
// direct-to-LDS load.
constexpr int PREFETCH_AHEAD = 1;
// LDS bytes past the two stages that absorb the prefetch loads' data.
constexpr int PREFETCH_SINK = 256;
// Then a double buffer of the tiles' targets (2 x 256 int32), and for the
// logit-gradient pass double buffers of their lse and upstream gradients
// (2 x 256 fp32 each).
constexpr int TGT_OFS = 4 * TILE_V * TILE_K * 2 + PREFETCH_SINK;
constexpr int LSE_OFS = TGT_OFS + 2 * TILE_T * 4;
constexpr int GRAD_OFS = LSE_OFS + 2 * TILE_T * 4;
// Then the two tile-claim slots of the dynamic walk.
constexpr int CLAIM_OFS = GRAD_OFS + 2 * TILE_T * 4;


__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base,
                                                            uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0,
                                           (int)bytes, RSRC_WORD3);
}

// Logical tile (token tile m, vocabulary tile n) of workgroup b.  The hardware
// deals workgroups to the 8 XCDs round-robin (b % 8); the first remap hands
// each XCD a contiguous run of logical tiles so that tiles sharing operands
// share one L2.  Within the logical order, GROUP_M token tiles advance through
// the vocabulary together, so a weight tile is read by all of them while it
// is hot.  Only the schedule changes; every tile's arithmetic is the same.
__device__ __forceinline__ void tile_of_block(int b, int nMT, int nVT, int &m,
                                              int &n) {
  const int total = nMT * nVT;
  const int per_xcd = total >> 3;
  int L = b;
  if (b < (per_xcd << 3)) L = (b & 7) * per_xcd + (b >> 3);
  const int in_group = GROUP_M * nVT;
  const int g = L / in_group;
  const int first_m = g * GROUP_M;
  const int gsm = min(nMT - first_m, GROUP_M);
  const int r = L - g * in_group;
  m = first_m + r % gsm;
  n = r / gsm;
}

// The same grouping for a logical tile index that is already XCD-ordered
// (the dynamic claims hand out logical indices directly).
__device__ __forceinline__ void tile_of_logical(int L, int nMT, int nVT, int &m, int &n) {
  const int in_group = GROUP_M * nVT;
  const int g = L / in_group;
  const int first_m = g * GROUP_M;
  const int gsm = min(nMT - first_m, GROUP_M);
  const int r = L - g * in_group;
  m = first_m + r % gsm;
  n = r / gsm;
}

// LDS layout of one operand stage: 256 rows x 64 bf16 (128 bytes per row);
// the 16-byte chunk c of row r sits at chunk position c ^ swz(r), where
// swz(r) = 4 r2 + r1 + 2 (r0 ^ r3) in the bits r3 r2 r1 r0 of r & 15.  A
// fragment read (ds_read_b128) has lanes 16 g + x on row x (16 consecutive
// rows) and chunk c0 + g.  The counters show the LDS serving lanes l and
// l + 32 in the same cycle: lanes x and x + 32 read one row's chunks c0 and
// c0 ^ 2.  swz maps each aligned octet of rows to 8 distinct positions, the
// even (and the odd) rows of an octet to four positions that differ in more
// than bit 1 (so chunks c and c ^ 2 of them never meet), and the 8 even (odd)
// rows of 16 to 8 distinct positions: the reads are free of bank conflicts
// whether the LDS serves 8 consecutive lanes (128-byte window), 16
// consecutive lanes, or lanes l .. l + 7 with l + 32 .. l + 39 (256-byte
// window) per cycle.
__device__ __forceinline__ int swz(int row) {
  return 4 * ((row >> 2) & 1) + ((row >> 1) & 1) + 2 * ((row & 1) ^ ((row >> 3) & 1));
}

// ds_read_b64_tr_b16 through a restrict-qualified pointer: inlined, the
// call then carries alias-scope information like the kernel's other LDS
// reads, and the compiler does not make it wait for every direct-to-LDS load
// in flight (without it, it waits with vmcnt(0) before each one).
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
__device__ __forceinline__ bf16x4 tr_read(const lds_bf16x4 *__restrict__ p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(const_cast<lds_bf16x4 *>(p));
}

// The logit GEMM with its epilogue, for a sequence of workgroup tiles of 256
// vocabulary x 256 token rows -- one tile shape for every batch size.  4
// waves; wave w covers vocabulary half wv = w & 1 and token half wt = w >> 1
// as 8 x 8 MFMA blocks of 16 x 16.  Every tile runs the same instructions:
// rows past T (in the last token tile of a batch whose size is not a
// multiple of 256, e.g. every decode batch) read as zeros through the buffer
// unit's range check, and no epilogue writes their results.  (Skipping their
// loads and MFMAs needs either a branch per load or MFMA, which measured 2.5 %
// slower on full tiles for the loads and 28 % for a branch inside each MFMA's
// assembly, or copies of the K loop specialised on the number of live rows,
// which push the option and backward epilogues into scratch spills and amount
// to a batch-size-dependent code path.)
//
// PERSIST: the workgroup walks tiles L = blockIdx.x, + gridDim.x, ... and
// issues the next tile's first K-block loads before the current tile's
// epilogue, so that their latency hides under the epilogue.  The order of
// tiles only changes the schedule; every tile's arithmetic is the same.
template <bool STATS, bool PERSIST, int EX, bool KMW>
__device__ __forceinline__ void gemm_body(const GemmArgs &a, char *smem) {
  static_assert(!(STATS && KMW), "the statistics pass reads K-contiguous operands");
  constexpr int NI = 8;         // vocabulary blocks of 16 rows per wave
  constexpr int NJ = 8;         // token blocks of 16 rows per wave
  constexpr int TT = 32 * NJ;   // token rows of a tile (TILE_T)
  constexpr int WT = 16 * NJ;   // token rows of a wave
  constexpr int NQ = NI * NJ;   // MFMAs per wave and 32-deep K step
  constexpr int BAR_Q = 40;     // the K block's barrier: behind this many MFMAs of step 1
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform
  const int wv = wave & 1;   // vocabulary half of the tile
  const int wt = wave >> 1;  // token half of the tile
  // Lane-dependent values (MFMA row lane & 15, K slice lane >> 4, load and
  // read offsets) are formed where they are used, from a fresh lane id, so
  // that none is live across both the K loop and the epilogue.

  const int total = a.nMT * a.nVT;
  // Dynamic tile claims (when the host passes a.queue):
  // the compute units do not run at one speed (per-XCD tile times differ by
  // several percent), so a fixed share of tiles per workgroup ends with the
  // slowest one.  Each XCD x claims the logical tiles of its own contiguous
  // range in order from counter a.queue[x] (the tiles that share weight tiles
  // in its L2 stay together), and once that range is exhausted takes tiles
  // from the other XCDs' ranges.  Thread 0 claims the next tile at the start
  // of the current one, just before the workgroup barrier there, and the
  // waves read it from LDS.  Which workgroup computes a tile changes no bit.
  const bool dyn = PERSIST && a.queue != nullptr;
  const int per_xcd = total >> 3;
  // two slots in the kernel's one LDS buffer (a separate __shared__ object
  // made the compiler wait for every direct-to-LDS load before LDS reads)
  int *claimed = reinterpret_cast<int *>(smem + CLAIM_OFS);
  auto claim = [&]() -> int {
    const int x = (int)(blockIdx.x & 7);
    for (int d = 0; d < 8; ++d) {
      const int y = (x + d) & 7;
      const int lo = y * per_xcd, hi = y == 7 ? total : lo + per_xcd;
      if (lo >= hi) continue;
      const int i = atomicAdd(&a.queue[y], 1);
      if (lo + i < hi) return lo + i;
    }
    return -1;
  };
  int L;
  if (dyn) {
    if (threadIdx.x == 0) claimed[0] = claim();
    __syncthreads();
    L = claimed[0];
    if (L < 0) return;
  } else {
    L = blockIdx.x;
    if (L >= total) return;
  }
  auto coords = [&](int l, int &m, int &n) {
    if (dyn) tile_of_logical(l, a.nMT, a.nVT, m, n);
    else tile_of_block(l, a.nMT, a.nVT, m, n);
  };

  // Global -> LDS: direct-to-LDS buffer loads (each lane's 16 bytes land in
  // LDS slot base + 16 * lane).  Load i of wave w fills the 1 KiB block
  // b = 4 i + w of a stage, i.e. rows 8 b .. 8 b + 7; lane l supplies row
  // 8 b + (l >> 3) and, because of the swizzle, global chunk
  // (l & 7) ^ swz(row) of that row.  The K
  // offset of the block rides in the scalar offset; rows past T or V fall
  // outside the tile's resource and read 0.
  //
  // A K-major weight-role operand ([depth][columns]; KMW) is handled by tile:
  // the tile's first column at depth row 0, the operand's rows along the
  // depth (kr), and the bytes from the tile's first column to the end of the
  // operand's last row.  Each K block reads through a resource of its own,
  // based at the block's first row (so no offset reaches 2^32 whatever the
  // operand's size) and ending at the operand's last element: depth rows
  // past kr read zeros, and so do the last row's columns past its end (kcols
  // columns, a multiple of 8, so that no 16-byte chunk is cut by the range
  // check, which drops each 4-byte piece on its own).  Columns past the end
  // in other rows read the next row's values; they only reach outputs of
  // columns past V, which are never stored.
  struct KMajor {
    const uint16_t *p;
    int krows;
    uint32_t cols;
  };
  using HW = std::conditional_t<KMW, KMajor, __amdgpu_buffer_rsrc_t>;
  auto rsrc_w = [&](int n) -> HW {
    const int v0 = n * TILE_V;
    if constexpr (KMW) {
      return KMajor{a.weight + v0, a.kr, (uint32_t)(a.kcols - v0) * 2u};
    } else {
      return make_rsrc(a.weight + (size_t)v0 * a.ldw,
                       (uint32_t)(min(TILE_V, a.V - v0) * a.ldw * 2));
    }
  };
  auto rsrc_h = [&](int m) {
    const int t0 = m * TT;
    return make_rsrc(a.hidden + (size_t)t0 * a.ldh,
                     (uint32_t)(min(TT, a.T - t0) * a.ldh * 2));
  };
  const __amdgpu_buffer_rsrc_t zero = make_rsrc(a.weight, 0u);
  auto zero_w = [&]() -> HW {
    if constexpr (KMW) return KMajor{a.weight, 0, 0u};
    else return zero;
  };
  // The resource and scalar offset through which K block kb of a tile's
  // weight-role operand is read.
  auto src_w = [&](HW h, int kb, uint32_t &so) -> __amdgpu_buffer_rsrc_t {
    if constexpr (KMW) {
      const int rows = min(TILE_K, h.krows - kb * TILE_K);
      so = 0;
      return make_rsrc(h.p + (size_t)kb * TILE_K * a.ldw,
                       rows > 0 ? (uint32_t)(rows - 1) * (uint32_t)a.ldw * 2u + h.cols : 0u);
    } else {
      so = (uint32_t)kb * (TILE_K * 2);
      return h;
    }
  };
  // token rows of tile m that lie below T
  auto rows_of = [&](int m) { return min(TT, a.T - m * TT); };
  uint32_t gofs[2][8];  // [operand][load]; set by set_offsets below
  typedef __attribute__((address_space(3))) void lds_void;
  // Load q (0..15) of K block kb into `stage`: the weight's row group q for
  // q < 8, then the hidden rows' group q - 8.  In the main loop the weight's
  // loads thus go out in the first K step and the hidden rows' in the second:
  // weight lines are the ones that miss L2 (streamed from HBM), and given the
  // longer head start the block ran 0.3-0.4 % faster than with the two
  // operands alternating (hidden rows first: 0.4 % slower; bitwise identical).
  // This wave's LDS slot; each K block makes it opaque to the compiler
  // (an empty asm), so the 32 destinations below are formed from it by
  // scalar adds where they are used instead of being held in 32 scalar
  // registers across the loop.
  typedef __attribute__((address_space(3))) char lds_char;
  lds_char *lds_wave = (lds_char *)smem + wave * 1024;
  // (r_w, s_w): the weight-role resource and scalar offset of the K block
  // being loaded (src_w); r_h the hidden-role tile's resource.
  auto gload = [&](__amdgpu_buffer_rsrc_t r_w, uint32_t s_w, __amdgpu_buffer_rsrc_t r_h,
                   int stage, int kb, int q) {
    const int op = q < 8 ? 0 : 1, i = q & 7;
    lds_char *dst = lds_wave + stage * (2 * STAGE_BYTES) + op * STAGE_BYTES + (4 * i) * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(op ? r_h : r_w, (lds_void *)dst, 16, gofs[op][i],
                                             op ? (uint32_t)kb * (TILE_K * 2) : s_w, 0, 0);
  };
  // L2 prefetch of the weight's K block kb: one 4-byte load per 128-byte
  // line, lane l touching row 32 (l >> 3) + 8 w + (l & 7) -- the 64 rows
  // this wave's own loads of that block will cover.  The data lands in a
  // scratch slot of LDS that nothing reads; the point is that the line is in
  // L2 when the real load comes PREFETCH_AHEAD blocks later.  Past the end of
  // a row or of the resource the load stays in bounds or reads nothing.
  // Only the weight is prefetched: it is streamed from HBM (far larger than
  // the last-level cache), while the hidden rows of a few token tiles stay
  // in the memory-side cache, where a prefetch costs the CU more in line
  // requests than it saves in latency (measured).
  uint32_t pofs_w, pofs_h;
  auto prefetch = [&](HW h, int kb) {
    uint32_t so;
    const __amdgpu_buffer_rsrc_t r = src_w(h, kb, so);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(smem + 4 * STAGE_BYTES), 4,
                                             pofs_w, so, 0, 0);
  };
  // The plain (store) GEMM also prefetches its hidden-role rows, the same
  // way, when pf_hidden is set (the backward's products, whose hidden-role
  // operand streams from HBM); otherwise through the zero-size resource.
  // Two prefetches in flight then, always, so the wait count is fixed.
  auto prefetch_h = [&](__amdgpu_buffer_rsrc_t r, int kb) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(smem + 4 * STAGE_BYTES), 4,
                                             pofs_h, (uint32_t)kb * (TILE_K * 2), 0, 0);
  };
  // A tile's first K block into stage 0, and its next blocks into L2.
  // Targets of a tile: one 4-byte direct-to-LDS load per wave (64 rows
  // each) into the tile's half of a double buffer, through a resource based
  // at the tile's first row and sized to its rows below T (rows past T read
  // 0; every offset stays below 1 KiB whatever T).  The logit-gradient pass
  // stages the rows' lse and upstream gradient the same way: read from LDS
  // in the epilogue, they hold no register across the K loop.
  // The lane offset is formed afresh (an asm the compiler cannot merge with
  // the set-up's): kept across the K loop it would be spilled, and its
  // reload would wait for every load in flight.
  auto stage_targets = [&](int tile_m, int par) {
    if (STATS) {
      int l;
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
      const uint32_t bytes = (uint32_t)(rows_of(tile_m) * 4);
      const int slot = par * (TILE_T * 4) + wave * 256;
      const __amdgpu_buffer_rsrc_t r_tgt = make_rsrc(a.targets + (size_t)tile_m * TT, bytes);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r_tgt, (lds_void *)(smem + TGT_OFS + slot), 4,
                                               (uint32_t)(l * 4), (uint32_t)(64 * wave * 4), 0,
                                               0);
      if constexpr (EX == 3) {
        const __amdgpu_buffer_rsrc_t r_lse = make_rsrc(a.lse + (size_t)tile_m * TT, bytes);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r_lse, (lds_void *)(smem + LSE_OFS + slot), 4,
                                                 (uint32_t)(l * 4), (uint32_t)(64 * wave * 4),
                                                 0, 0);
        const __amdgpu_buffer_rsrc_t r_g = make_rsrc(a.grad + (size_t)tile_m * TT, bytes);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r_g, (lds_void *)(smem + GRAD_OFS + slot), 4,
                                                 (uint32_t)(l * 4), (uint32_t)(64 * wave * 4),
                                                 0, 0);
      }
    }
  };
  auto issue_first = [&](HW r_w, __amdgpu_buffer_rsrc_t r_h, HW p_w,
                         __amdgpu_buffer_rsrc_t p_h) {
    uint32_t s_w;
    const __amdgpu_buffer_rsrc_t b_w = src_w(r_w, 0, s_w);
#pragma unroll
    for (int q = 0; q < 16; ++q) gload(b_w, s_w, r_h, 0, 0, q);
#pragma unroll
    for (int kp = 1; kp <= PREFETCH_AHEAD; ++kp) {
      prefetch(p_w, kp);
      if constexpr (!STATS) prefetch_h(p_h, kp);
    }
  };

  // MFMA v_mfma_f32_16x16x32_bf16: a 16 x 16 block of outputs from 16
  // A rows and 16 B rows over 32 K.  Lane l supplies 8 consecutive K
  // values, 8 (l >> 4) .. + 7, of A row l & 15 and of B row l & 15, and
  // receives outputs (A row 4 (l >> 4) + r, B row l & 15), r = 0 .. 3.
  // Each wave covers its 128 x 128 outputs as 8 x 8 such blocks.
  //
  // Fragment reads: A (weight) rows wv*128 + 16 i + (l & 15), B (hidden)
  // rows wt*128 + 16 j + (l & 15), 16-byte chunk 4 s + (l >> 4) of K step s
  // (0, 1) of the 64-wide block.  swz(16 i + x) == swz(x), so the byte
  // address is a lane base per (stage, s) plus i * 2048.
  //
  // A K-major weight stage holds 64 depth rows k x 256 columns c (32 chunks
  // of 8 columns) as 128 lines of 256 bytes: chunk c of row k sits in line
  // 8 (k >> 2) + (c >> 2), 16-byte slot 2 (k & 3) + (c & 1) +
  // 8 (((c >> 1) & 1) ^ ((k >> 3) & 1)).  The MFMA operand of a 16-column
  // block and a 32-deep K step is two transposing reads (ds_read_b64_tr_b16:
  // in each group of 16 lanes, lane 4 r + s supplies columns 4 s .. 4 s + 3
  // of row r, and lane i receives column i of the 4 rows): the lanes of
  // group g = l >> 4 read rows 32 s + 8 g + 4 h + 0 .. 3 (h = 0, 1) as one
  // contiguous 128-byte piece, at lane base + 16384 s + 2048 h + 256 (i >> 1)
  // (immediate offsets; the base differs by the parity of i).  The XOR with
  // (k >> 3) & 1 puts groups g and g + 1 in different halves of a 256-byte
  // bank window, so each read is free of bank conflicts.  Load i of wave w
  // fills lines 4 b .. 4 b + 3, b = 4 i + w (rows 8 i + 4 (w >> 1) .. + 3,
  // 256 contiguous bytes of each): lane l fetches row 8 i + 4 (w >> 1) +
  // ((l >> 1) & 3), chunk 16 (w & 1) + 4 (l >> 4) + 2 (((l >> 3) & 1) ^
  // (i & 1)) + (l & 1).
  uint32_t ra[2][2], rb[2][2];
  uint32_t kma[2][2];   // K-major weight: lane base per stage and parity of i
  // The per-lane offsets of the loads, the prefetch and the fragment reads,
  // formed at the start of every tile from a lane id the compiler cannot
  // merge with an earlier one: they are then dead during the epilogue
  // instead of held (or spilled and reloaded) across it.
  auto set_offsets = [&]() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    const int lrow = 8 * wave + (l >> 3);
    const int lchunk = (l & 7) ^ swz(lrow);   // swz(lrow + 32 i) == swz(lrow)
    const int kmrow = 4 * (wave >> 1) + ((l >> 1) & 3);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int kmchunk =
          16 * (wave & 1) + 4 * (l >> 4) + 2 * (((l >> 3) & 1) ^ (i & 1)) + (l & 1);
      gofs[0][i] = KMW ? (uint32_t)((8 * i + kmrow) * a.ldw * 2 + kmchunk * 16)
                       : (uint32_t)((lrow + 32 * i) * a.ldw * 2 + lchunk * 16);
      gofs[1][i] = (uint32_t)((lrow + 32 * i) * a.ldh * 2 + lchunk * 16);
    }
    // L2 prefetch; K-major: row 16 w + (l >> 2), 128-byte line l & 3
    const int prow = 32 * (l >> 3) + 8 * wave + (l & 7);
    pofs_w = KMW ? (uint32_t)((16 * wave + (l >> 2)) * a.ldw * 2 + (l & 3) * 128)
                 : (uint32_t)(prow * a.ldw * 2);
    pofs_h = (uint32_t)(prow * a.ldh * 2);
    const int lr = l & 15, lg = l >> 4;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int ip = 0; ip < 2; ++ip)
        kma[st][ip] = st * (2 * STAGE_BYTES) + 4096 * lg + 1024 * wv + 8 * lr +
                      128 * (ip ^ (lg & 1));
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const uint32_t x = (uint32_t)(((4 * ks + lg) ^ swz(lr)) << 4);
        ra[st][ks] = st * (2 * STAGE_BYTES) + (wv * 128 + lr) * 128 + x;
        rb[st][ks] = st * (2 * STAGE_BYTES) + STAGE_BYTES + (wt * WT + lr) * 128 + x;
      }
    }
  };
  // A fragments: one set, each refilled for the next K step once its own
  // MFMAs are issued; B fragments: two sets, one per K step.
  bf16x8 fa[NI], fb[2][NJ];
  // A fragment, block i of K step ks (K-major: two transposing reads)
  auto reada = [&](int st, int ks, int i) {
    if constexpr (KMW) {
      lds_char *p = (lds_char *)smem + kma[st][i & 1] + 16384 * ks + 256 * (i >> 1);
      const bf16x4 lo = tr_read((const lds_bf16x4 *)p);
      const bf16x4 hi = tr_read((const lds_bf16x4 *)(p + 2048));
      fa[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    } else {
      fa[i] = *(const bf16x8 *)(smem + ra[st][ks] + i * 2048);
    }
  };
  auto readb = [&](int buf, int st, int ks, int j) {
    fb[buf][j] = *(const bf16x8 *)(smem + rb[st][ks] + j * 2048);
  };
  f32x4 acc[NI][NJ];
  // MFMA q of a K step: A block i = q / 8 with the eight B blocks in turn,
  // so A_i is used by MFMAs 8 i .. 8 i + 7 (an operand held for eight
  // MFMAs in a row toggles the matrix core's inputs less: measured, the
  // clock the kernel holds at the power limit is ~1.5 % higher than with A
  // held for four).  The B blocks go up for even i and down for odd i, so
  // the MFMA that moves on to the next A block keeps the B operand of the
  // one before it (~0.5 % faster, same reason).  Each accumulator still
  // takes its K steps in K order, so the sums are the same bits either way.
  // In inline assembly: the builtin of this instruction gets its
  // accumulator copied between registers on every use by this compiler,
  // while the assembly form keeps each accumulator in place.  The compiler
  // does not see an MFMA here, so the tile supplies the wait states it
  // would insert (after zeroing the accumulators and before reading them,
  // below).
  auto mfma = [&](int buf, int q) {
    const int i = q >> 3, j = (i & 1) ? 7 - (q & 7) : (q & 7);
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                 : "+a"(acc[i][j])
                 : "v"(fa[i]), "v"(fb[buf][j]));
  };

  // One K block of the main loop: two 32-deep K steps of 64 MFMAs.  Each
  // accumulator advances in increasing k (32 per MFMA); the fixed
  // instruction order below only decides what overlaps with what.  The
  // fragment reads are spread one per two to four MFMAs (a burst of them
  // queues in the LDS, and the MFMAs wait):
  //   Step 0 (B set 0): behind MFMAs 1, 5, 9, 13 this step's A_4-7 (the
  //   block before read only what its first MFMAs need); behind 17, 21, ..,
  //   45 step 1's B_0-7 (set 1); behind 8 i + 10 (i < 6) and 58 step 1's
  //   A_i, i < 7 (each after its last use here, MFMA 8 i + 7); behind every
  //   third MFMA (1, 4, .., 46) one direct-to-LDS load of the next K block,
  //   so the sixteen loads are issued early (the barrier that waits for them
  //   comes 1.5 steps later) but never in bursts (a burst stalls the wave's
  //   in-order issue, and with it the next MFMA, until the texture path
  //   takes the load).
  //   Step 1 (B set 1): behind MFMA 2 its A_7, behind 16 the L2 prefetch;
  //   after MFMA BAR_Q - 1 (39) the wave waits for its loads and the
  //   workgroup meets at the barrier (the next block has landed; this block
  //   is no longer read); then behind the 15 MFMAs after it the next
  //   block's B_0-7 (set 0, every second one) and A_0-3 (every fourth; last
  //   used here at MFMA 31 or before).  (Barrier positions 32, 40 and 48
  //   measured the same at 4096 rows; 40 and 48 hide more of the weight
  //   stream's latency at 256 rows.)
  // The loads fetch K block kl of (r_w, r_h) into the other stage: kb + 1
  // of this tile, and in the tile's last block block 0 of the next tile
  // (r_w, r_h then name the next tile; the other stage is free once the
  // barrier of the block before has passed).  p_w and kp name the weight
  // block the L2 prefetch fetches: kb + 1 + PREFETCH_AHEAD of this tile, and
  // in the last two blocks the next tile's blocks 0 and 1.  Every block,
  // the last included, meets the barrier and reads the next block's first
  // fragments (in the last block those of the next tile's first block, which
  // the next tile reads again after its epilogue).
  auto k_block = [&](int kb, auto stage, int kl, HW r_w, __amdgpu_buffer_rsrc_t r_h, HW p_w,
                     __amdgpu_buffer_rsrc_t p_h, int kp, bool sync) {
    constexpr int st = decltype(stage)::value;    // == kb & 1
    uint32_t s_w;
    const __amdgpu_buffer_rsrc_t b_w = src_w(r_w, kl, s_w);
    asm volatile("" : "+s"(lds_wave));
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      mfma(0, q);
      if (q < 16 && (q & 3) == 1) reada(st, 0, 4 + (q >> 2));
      if (q >= 17 && q <= 45 && (q & 3) == 1) readb(1, st, 1, (q - 17) >> 2);
      if (q >= 10 && q <= 50 && (q & 7) == 2) reada(st, 1, (q - 10) >> 3);
      if (q == 58) reada(st, 1, 6);
      if (q < 48 && q % 3 == 1) gload(b_w, s_w, r_h, st ^ 1, kl, q / 3);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int q = 0; q < BAR_Q; ++q) {
      mfma(1, q);
      if (q == 2) reada(st, 1, 7);
      if (q == 16) {
        prefetch(p_w, kp);
        if constexpr (!STATS) prefetch_h(p_h, kp);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // This wave's loads of the next block have landed (only the prefetch
    // issued after them may still be in flight) and its reads of this block
    // are complete; then the workgroup barrier.  A plain s_barrier, not a
    // fenced __syncthreads(), so that the prefetch is not waited for; the
    // empty asm statements keep the compiler from moving memory accesses
    // across it.  The tile's last block (sync false) skips both: its loads
    // (the next tile's first block) are waited for after the epilogue, at
    // the next tile's start, so that their latency hides under the
    // epilogue, and what it reads below is read again there.
    asm volatile("" ::: "memory");
    if (sync) {
      __builtin_amdgcn_s_waitcnt(STATS ? VMCNT1_LGKMCNT0 : VMCNT2_LGKMCNT0);
      __builtin_amdgcn_s_barrier();
    }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int q = BAR_Q; q < NQ; ++q) {
      mfma(1, q);
      if (q > BAR_Q && q < BAR_Q + 16 && ((q - BAR_Q) & 1) == 1)
        readb(0, st ^ 1, 0, (q - BAR_Q - 1) >> 1);
      if (q > BAR_Q && q < BAR_Q + 16 && ((q - BAR_Q) & 3) == 2)
        reada(st ^ 1, 0, (q - BAR_Q - 2) >> 2);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // K blocks are run in pairs (stage 0, stage 1).  When H / 64 is odd, one
  // more block is appended whose loads go through a resource of zero size:
  // it reads zeros and adds exact zero products (it can only turn a logit
  // of -0 into +0, the same way for every row of a given H).
  const int nk = a.H / TILE_K;
  const int nk2 = nk + (nk & 1);
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;

  // The GROUP_M = 4 workgroups that share a weight tile run side by side on
  // one XCD (token tiles 4g .. 4g + 3); each prefetches one quarter of the
  // tile's rows, the quarter of its wave number m & 3, so every line is
  // requested once per group instead of four times.  The other waves
  // prefetch through the zero-size resource (no memory access).  A group
  // with fewer token tiles (fewer than 4 in all, or the last group) keeps
  // the whole prefetch in every workgroup.
  auto pf_rsrc = [&](int mm, HW r) -> HW {
    const bool full_group = (mm & ~(GROUP_M - 1)) + GROUP_M <= a.nMT;
    return (!full_group || wave == (mm & (GROUP_M - 1))) ? r : zero_w();
  };
  static_assert(GROUP_M == GEMM_THREADS / 64, "one prefetching wave per group member");
  int m, n;
  coords(L, m, n);
  HW rw = rsrc_w(n);
  __amdgpu_buffer_rsrc_t rh = rsrc_h(m);
  HW pw = pf_rsrc(m, rw);
  auto pfh_rsrc = [&](__amdgpu_buffer_rsrc_t r) { return a.pf_hidden ? r : zero; };
  __amdgpu_buffer_rsrc_t ph = pfh_rsrc(rh);
  int parity = 0;
  set_offsets();
  stage_targets(m, 0);
  issue_first(rw, rh, pw, ph);

  for (;;) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    set_offsets();
    if (dyn && threadIdx.x == 0) claimed[parity ^ 1] = claim();   // the next tile
    // The tile's first block (issued by the previous tile's last K block, or
    // above).
    __builtin_amdgcn_s_waitcnt(VMCNT0);
    __syncthreads();
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      if (x < 4) reada(0, 0, x);
      readb(0, 0, 0, x);
    }
    // Wait states between the accumulators' zeroing (VALU writes) and the
    // first MFMA that reads them.
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 4");
    __builtin_amdgcn_sched_barrier(0);
    // The next tile (scalars; its resources are formed in the last K pair).
    const int Ln = dyn ? claimed[parity ^ 1] : PERSIST ? L + (int)gridDim.x : total;
    const bool more_tiles = dyn ? Ln >= 0 : Ln < total;
    int mn = m, nn = n;
    if (more_tiles) coords(Ln, mn, nn);
    // Every K block in one loop (no copy of the K-block code after it: the
    // register copies a compiler may place between such copies would sit
    // next to MFMAs whose wait states it does not know about).  K blocks run
    // in pairs (stage 0, stage 1).  In the last pair the loads of the second
    // block (a zero block when H / 64 is odd) and of the next tile's first
    // block, and the L2 prefetches of the next tile's first two weight
    // blocks, take their resources from the next tile (after the last tile,
    // the zero-size resource: they read nothing).
    for (int kb = 0; kb < nk2; kb += 2) {
      const bool last = kb + 2 == nk2;
      HW w0 = rw, w1 = rw, p = pw;
      __amdgpu_buffer_rsrc_t h0 = rh, h1 = rh, ph_ = ph;
      int kp0 = kb + 1 + PREFETCH_AHEAD, kp1 = kb + 2 + PREFETCH_AHEAD, kl1 = kb + 2;
      if (last) {
        w1 = more_tiles ? rsrc_w(nn) : zero_w();
        h1 = more_tiles ? rsrc_h(mn) : zero;
        p = pf_rsrc(mn, w1);
        ph_ = pfh_rsrc(h1);
        if (nk & 1) {
          w0 = zero_w();
          h0 = zero;
        }
        kp0 = 0;
        kp1 = 1;
        kl1 = 0;
      }
      k_block(kb, S0{}, kb + 1, w0, h0, p, ph_, kp0, true);
      if (last) stage_targets(mn, parity ^ 1);   // after the last tile: its own, unused
      // (the logit-gradient pass keeps the wait: without it the pass
      // measured no faster, with its heavier epilogue of stores)
      k_block(kb + 1, S1{}, kl1, w1, h1, p, ph_, kp1, !last || EX == 3);
      // wait states after the iteration's last MFMA, for register copies
      // the compiler may place where the loop ends (issued while the MFMA
      // pipeline is still busy)
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_nop 7\n\ts_nop 3");
      __builtin_amdgcn_sched_barrier(0);
    }
    // Wait states between the last MFMA and the first read of its result
    // (more than the instruction's latency requires).
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
    __builtin_amdgcn_sched_barrier(0);

    const int v0 = n * TILE_V;
    const int t0 = m * TT;
    // The epilogue's lane values, computed afresh (an asm the compiler cannot
    // merge with the set-up's) so that nothing from the set-up stays live
    // across the K loop or is spilled: a reload from scratch here would be
    // a vector memory op, and waiting for it would also wait for the next
    // tile's loads issued by the last K block.
    int lane_e;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane_e));

    // acc[i][j][r] holds z[t][v] for
    //   v = v0 + wv*128 + 16 i + 4 fg + r
    //   t = t0 + wt*WT + 16 j + fc
    const int vbase = v0 + wv * 128;
    {
    const int fc = lane_e & 15;
    const int fg = lane_e >> 4;
    // Combining the four row groups' values of a column (lanes fc, fc + 16,
    // fc + 32, fc + 48) in the VALU: v_permlane16_swap exchanges the odd
    // 16-lane rows of one copy with the even rows of the other, so the pair
    // (lo, hi) below holds, in every lane, the values of rows 2 k and 2 k + 1
    // of its pair of rows; v_permlane32_swap does the same for the halves.
    // Every lane then applies the operation in the same operand order.
    auto rows16 = [](float x, float &lo, float &hi) {
      const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                      false, false);
      lo = __uint_as_float(r[0]);
      hi = __uint_as_float(r[1]);
    };
    auto rows32 = [](float x, float &lo, float &hi) {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                      false, false);
      lo = __uint_as_float(r[0]);
      hi = __uint_as_float(r[1]);
    };
    // the register of a 16-row block that holds row rel (0 .. 127) for the
    // lane of row group (rel >> 2) & 3: block rel >> 4, register rel & 3,
    // picked by a fixed select tree over the 32 values of token block j
    auto pick = [&](int j, int rel) {
      const int bi = (rel >> 4) & 7, ri = rel & 3;
      float sel[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v8[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v8[i] = acc[i][j][r];
#pragma unroll
        for (int lvl = 0; lvl < 3; ++lvl) {
          const bool bit = (bi >> lvl) & 1;
#pragma unroll
          for (int q = 0; q < (4 >> lvl); ++q) v8[q] = bit ? v8[2 * q + 1] : v8[2 * q];
        }
        sel[r] = v8[0];
      }
      const float lo = (ri & 1) ? sel[1] : sel[0];
      const float hi = (ri & 1) ? sel[3] : sel[2];
      return (ri & 2) ? hi : lo;
    };
    // this tile's targets, staged in LDS before its K loop (read with
    // ds_read: no wait on the vector memory counter)
    const int *tgt = reinterpret_cast<const int *>(smem + TGT_OFS + parity * (TILE_T * 4));
    const float *lse_s = reinterpret_cast<const float *>(smem + LSE_OFS + parity * (TILE_T * 4));
    const float *grad_s = reinterpret_cast<const float *>(smem + GRAD_OFS + parity * (TILE_T * 4));
    auto target_of = [&](int j, int t) {
      return (t < a.T) ? tgt[wt * WT + 16 * j + fc] : -1;
    };
    // neighbouring-lane exchange (lane l gets lane l ^ 1's value): a DPP quad
    // permutation [1, 0, 3, 2] in the VALU, no LDS round trip
    auto xor1i = [&](int x) { return __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false); };
    if constexpr (!STATS) {
      // Registers 4q .. 4q+3 hold four consecutive columns.  Stores are raw
      // buffer stores over one resource per 32-row group (at most 32 V
      // floats: the host keeps V <= 2^24, so the size fits 2^31 bytes).  A
      // row past T lies past the resource's size, and a column past V is
      // given offset 2^31, so the hardware's range check drops both stores:
      // no branch per element.  With V a multiple of 4 and a 16-byte aligned
      // output (EX == 0) the rows go through LDS and leave as whole rows, four
      // columns per lane; otherwise (EX == 1, chosen by the host) one column
      // per store straight from the accumulators.  The two are separate
      // instantiations; the arithmetic, and so every stored bit, is the same.
      constexpr uint32_t DROP = 0x80000000u;
      constexpr bool vec = EX == 0;
      if constexpr (EX == 2) {
        // Transposed: out[v][t], row stride T.  Each wave stages 32 of its
        // 128 weight-role rows v at a time (blocks i = 2 ip, 2 ip + 1; 32 x
        // 128 fp32, 16 KiB) in its quarter of the operand buffer's stage 1,
        // staging row R = 16 ii + 4 fg + r holding the wave's 128 columns t,
        // then stores whole 512-byte row pieces, two rows per instruction.
        // A lane's four registers of a block are four rows of one column, so
        // the writes are single dwords.  16-byte chunk c of staging row R
        // sits at slot c ^ 4 ((R >> 2) & 3) ^ (R & 1): the four row groups
        // of a write fall in different banks, and so do the two rows of a
        // read (lanes l and l + 32).
        typedef __attribute__((address_space(3))) char lds_c;
        lds_c *stg = (lds_c *)smem + 2 * STAGE_BYTES + wave * (STAGE_BYTES / 2);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        const int u = lane_e & 31, rh = lane_e >> 5;
        const int tcol = t0 + wt * WT + 4 * u;   // this lane's first column
        const uint32_t coff = tcol < a.T ? 4u * (uint32_t)tcol : DROP;
#pragma unroll
        for (int ip = 0; ip < NI / 2; ++ip) {
#pragma unroll
          for (int ii = 0; ii < 2; ++ii)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                // R = 16 ii + 4 fg + r: (R >> 2) & 3 == fg, R & 1 == r & 1
                const int slot = (4 * j + (fc >> 2)) ^ (4 * fg) ^ (r & 1);
                *(uint32_t *)(stg + (16 * ii + 4 * fg + r) * 512 + (slot << 4) + 4 * (fc & 3)) =
                    __float_as_uint(acc[2 * ip + ii][j][r]);
              }
          const int vrow = vbase + 32 * ip;
          const int rows = min(32, a.V - vrow);
          const __amdgpu_buffer_rsrc_t r_out =
              make_rsrc(a.logits + (size_t)vrow * a.T,
                        rows > 0 ? (uint32_t)rows * (uint32_t)a.T * 4u : 0u);
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int R = 2 * e + rh;
            const int slot = u ^ (4 * ((R >> 2) & 3)) ^ (R & 1);
            const u32x4 d = *(const u32x4 *)(stg + R * 512 + (slot << 4));
            const uint32_t off = coff == DROP ? DROP : (uint32_t)R * (uint32_t)a.T * 4u + coff;
            __builtin_amdgcn_raw_buffer_store_b128(d, r_out, (int)off, 0, 0);
          }
        }
      } else if constexpr (vec) {
        // Through LDS: each wave stages 32 token rows at a time (two token
        // blocks; 32 rows x 128 columns fp32, 16 KiB) in its quarter of the
        // operand buffer's stage 1 (free once every wave is past the tile's
        // last K block), then stores whole rows, two per instruction: 8 full
        // lines per store instead of 32 rows x 32 bytes.  16-byte chunk c of
        // staging row r sits at slot c ^ (r & 15), which keeps the writes (16
        // rows, one chunk) and the row reads free of bank conflicts.
        typedef __attribute__((address_space(3))) char lds_c;
        lds_c *stg = (lds_c *)smem + 2 * STAGE_BYTES + wave * (STAGE_BYTES / 2);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
#pragma unroll
        for (int jp = 0; jp < NJ / 2; ++jp) {
#pragma unroll
          for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int i = 0; i < NI; ++i) {
              const f32x4 v = acc[i][2 * jp + jj];
              *(u32x4 *)(stg + (16 * jj + fc) * 512 + (((4 * i + fg) ^ fc) << 4)) =
                  u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                        __float_as_uint(v[3])};
            }
          const int trow = t0 + wt * WT + 32 * jp;
          const int rows = min(32, a.T - trow);
          const __amdgpu_buffer_rsrc_t r_out = make_rsrc(
              a.logits + (size_t)trow * a.V, rows > 0 ? (uint32_t)rows * (uint32_t)a.V * 4u : 0u);
          // row r = 2 e + (lane >> 5), columns 4 u .. 4 u + 3, u = lane & 31
          const int u = lane_e & 31, rh = lane_e >> 5;
          const int v4 = vbase + 4 * u;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int r = 2 * e + rh;
            const u32x4 d = *(const u32x4 *)(stg + r * 512 + ((u ^ (r & 15)) << 4));
            const uint32_t off =
                v4 < a.V ? (uint32_t)r * (uint32_t)a.V * 4u + 4u * (uint32_t)v4 : DROP;
            __builtin_amdgcn_raw_buffer_store_b128(d, r_out, (int)off, 0, 0);
          }
        }
      } else {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int trow = t0 + wt * WT + 16 * j;
        const int rows = min(16, a.T - trow);
        const __amdgpu_buffer_rsrc_t r_out = make_rsrc(
            a.logits + (size_t)trow * a.V, rows > 0 ? (uint32_t)rows * (uint32_t)a.V * 4u : 0u);
        const uint32_t rofs = (uint32_t)fc * (uint32_t)a.V * 4u;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int v4 = vbase + 16 * i + 4 * fg;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int v = v4 + rr;
            const uint32_t off = v < a.V ? rofs + 4u * (uint32_t)v : DROP;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][rr]), r_out,
                                                  (int)off, 0, 0);
          }
        }
      }
      }  // vec
    } else {
      // Statistics tiles are 128 vocabulary rows wide: wave (wv, wt) owns
      // tile js = 2 n + wv (of this weight slice; js_base + js globally) for
      // its 128 token rows, so no data crosses waves.
      // A wave whose tile starts at or past V (only in the last workgroup
      // column when V mod 256 <= 128) has nothing to write.
      const int js = 2 * n + wv;
      if constexpr (EX == 3) {
        // The backward's logit gradient.  The logits are the forward's bits
        // (same main loop, same 1/tau multiply); with the forward's lse,
        // p = exp(z' - lse) and dz = g inv_tau (1[v == y] - p), in fp32, then
        // rounded to bf16 (nearest, ties to even) as the operand of the two
        // gradient GEMMs.  Rows past T, columns past V and rows whose target
        // is outside [0, V) hold 0.
        //
        // Each wave stages its 128 x 128 block of dz, 64 token rows at a
        // time, in 16 KiB of the operand buffer's stage 1 (free once every
        // wave is past the tile's last K block; the next tile's first block
        // lands in stage 0), then writes dz [T][ld_dz] as 16-byte row
        // pieces: 32 full stores per wave and tile instead of 128 narrow
        // scattered ones.  (The product over the tokens reads dz K-major as
        // stored, so no transposed copy is written.)  Staging row r holds
        // the 128 columns as 32 chunks of 4 (8 bytes); chunk c sits at slot
        // c ^ sw(r), sw(r) = 4 (r & 3) + ((r >> 2) & 3), which keeps the
        // writes (16 rows, one chunk) and the row reads (one row, 16 x 16
        // bytes) free of bank conflicts.  Pass p stages token blocks 4 p ..
        // 4 p + 3: block jj of the pass in staging rows 16 jj .. 16 jj + 15.
        typedef __attribute__((address_space(3))) char lds_c;
        lds_c *stg = (lds_c *)smem + 2 * STAGE_BYTES + wave * (STAGE_BYTES / 2);
        auto sw = [](int r) { return ((r & 3) << 2) | ((r >> 2) & 3); };
        auto slot = [&](int r, int c) { return stg + r * 256 + ((c ^ sw(r)) << 3); };
        // every wave's fragment reads of stage 1 are done
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        // Writing one staging pass.  Every column first gets g inv_tau (0 - p);
        // a dead row (past T, or target outside [0, V)) is cleared on the
        // packed bf16 bits, columns past V only in the vocabulary-tail copy
        // (MASK), and the one column v == y of a live row is then rewritten
        // with g inv_tau (1 - p) by the lane that holds it.  The values are
        // those of forming g inv_tau (1[v == y] - p) per column: 0 - p and
        // 1 - p are the same subtractions, a cleared value is +0.
        auto stage_pass = [&](int p, auto masked) {
          constexpr bool MASK = decltype(masked)::value;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int j = 4 * p + jj;
            const int t = t0 + wt * 128 + 16 * j + fc;
            const bool trow = t < a.T;
            const int y = trow ? target_of(j, t) : -1;
            const bool live = trow && y >= 0 && y < a.V;
            const float lse_t = live ? lse_s[wt * WT + 16 * j + fc] : 0.0f;
            const float gs = live ? grad_s[wt * WT + 16 * j + fc] * a.inv_tau : 0.0f;
            const uint64_t keep = live ? ~0ull : 0ull;
            const int lim = a.V - vbase - 4 * fg;   // MASK: offsets below lim are valid
#pragma unroll
            for (int i = 0; i < NI; ++i) {
              uint16_t b[4];
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) {
                const float zs = acc[i][j][rr] * a.inv_tau;
                const float pr = __builtin_amdgcn_exp2f((zs - lse_t) * LOG2E);
                float d = gs * (0.0f - pr);
                if (MASK && 16 * i + rr >= lim) d = 0.0f;
                b[rr] = __builtin_bit_cast(uint16_t, (__bf16)d);
              }
              const uint64_t packed = (uint64_t)b[0] | ((uint64_t)b[1] << 16) |
                                      ((uint64_t)b[2] << 32) | ((uint64_t)b[3] << 48);
              *(uint64_t *)slot(16 * jj + fc, 4 * i + fg) = packed & keep;
            }
            // the target column: block rel >> 4, register rel & 3, in the
            // lane of row group (rel >> 2) & 3
            const int rel = y - vbase;
            const bool hit = live && rel >= 0 && rel < STAT_V && ((rel >> 2) & 3) == fg;
            if (__any(hit)) {
              const float zy = pick(j, rel);
              if (hit) {
                const float zs = zy * a.inv_tau;
                const float pr = __builtin_amdgcn_exp2f((zs - lse_t) * LOG2E);
                const float d = gs * (1.0f - pr);
                *(uint16_t *)(slot(16 * jj + fc, (rel & (STAT_V - 1)) >> 2) + 2 * (rel & 3)) =
                    __builtin_bit_cast(uint16_t, (__bf16)d);
              }
            }
          }
        };
        const bool tail = n == a.nVT - 1 && a.V % TILE_V != 0;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          if (tail) stage_pass(p, std::true_type{});
          else stage_pass(p, std::false_type{});
          // The wave reads back only what it wrote, and LDS executes a wave's
          // accesses in issue order: no wait between the writes and the reads,
          // nor before the next pass overwrites the rows.
          const int trow0 = t0 + wt * 128 + 64 * p;   // token of staging row 0
          if (a.dz) {
            // row r = 4 e + (lane >> 4), columns 8 u .. 8 u + 7, u = lane & 15:
            // chunks 2u, 2u + 1 share one 16-byte slot, swapped when sw(r) is odd
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int r = 4 * e + (lane_e >> 4), u = lane_e & 15;
              // the even slot of the pair: 16-byte aligned
              const u32x4 d = *(const u32x4 *)(stg + r * 256 + ((2 * u ^ (sw(r) & ~1)) << 3));
              const bool swp = sw(r) & 1;
              const u32x4 o = swp ? u32x4{d[2], d[3], d[0], d[1]} : d;
              const int t = trow0 + r, v = vbase + 8 * u;
              if (t < a.T && v < a.Vp) *(u32x4 *)(a.dz + (size_t)t * a.ld_dz + v) = o;
            }
          }
        }
      } else {
      // The options, applied to each logit where it is read (the same fp32
      // multiply, exact for inv_tau == 1, then the fp32 -> bf16 cast,
      // nearest, ties to even): the same values as rewriting the
      // accumulators once, without the register pressure of writing back.
      const float itau = a.inv_tau;
      const bool rb16 = a.bf16_logits != 0;
      auto xf = [&](float z) {
        if constexpr (EX == 1 || EX == 2) {
          z = z * itau;
          if (rb16) z = (float)(__bf16)z;
        }
        return z;
      };
      auto stats_epilogue = [&](auto masked) {
        constexpr bool MASK = decltype(masked)::value;
        // Columns past the vocabulary end count as -inf: they add nothing to
        // the max and exactly 0 to the sum.  On valid columns the masked and
        // unmasked instantiations compute the same thing.
        const int lim = a.V - vbase - 4 * fg;  // columns at offset < lim are valid
        auto zv = [&](int i, int j, int r) {
          const bool out = MASK && (16 * i + r >= lim);
          return out ? -INFINITY : xf(acc[i][j][r]);
        };
        // Token blocks two at a time (one with 1/tau and bf16 rounding alone:
        // two spilled 38 registers there, one spills 6), with no branch until
        // the stores (so the blocks' dependency chains overlap).
        constexpr int JG = EX == 0 ? 2 : 1;
        // 1) tile max: this lane's 32 values in (i, r) order, then across
        //    the four lanes (row groups fg) holding the tile's 128 rows:
        //    row groups 0 with 1 and 2 with 3, then the two pairs.
        // 2) sum of exp(z - m): the lane's 32 exponentials added as a fixed
        //    pairwise tree ((e0 + e1) + (e2 + e3)) + ..., in (i, r) order
        //    (subtrees of 4 per block i, then those eight pairwise),
        //    then across the row groups as for the max; m is taken as 0 when
        //    the whole tile is -inf so that such a tile adds exactly 0.  z == m
        //    gives exp(0) = 1 exactly, so the sum is >= 1 when the max is
        //    finite.  The entropy partial e (z - m) the same way (a -inf
        //    logit has e == 0 and adds -0: d clamped to the finite range).
        float m2[NJ], s2[NJ], u2[NJ];
#pragma unroll
        for (int jg = 0; jg < NJ; jg += JG) {
#pragma unroll
          for (int j = jg; j < jg + JG; ++j) {
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < NI; ++i)
#pragma unroll
              for (int r = 0; r < 4; ++r) mx = fmaxf(mx, zv(i, j, r));
            m2[j] = mx;
          }
#pragma unroll
          for (int j = jg; j < jg + JG; ++j) {
            float lo, hi;
            rows16(m2[j], lo, hi);
            const float m1 = fmaxf(lo, hi);
            rows32(m1, lo, hi);
            m2[j] = fmaxf(lo, hi);
          }
#pragma unroll
          for (int j = jg; j < jg + JG; ++j) {
            const float ms = (m2[j] == -INFINITY) ? 0.0f : m2[j];
            float ps[8], pu[8];
#pragma unroll
            for (int i = 0; i < NI; ++i) {
              float e[4], u[4];
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const float d = zv(i, j, r) - ms;
                e[r] = __builtin_amdgcn_exp2f(d * LOG2E);
                if constexpr (EX == 2) u[r] = e[r] * fmaxf(d, -FLT_MAX);
              }
              ps[i] = (e[0] + e[1]) + (e[2] + e[3]);
              if constexpr (EX == 2) pu[i] = (u[0] + u[1]) + (u[2] + u[3]);
            }
            s2[j] = ((ps[0] + ps[1]) + (ps[2] + ps[3])) + ((ps[4] + ps[5]) + (ps[6] + ps[7]));
            u2[j] = EX == 2
                        ? ((pu[0] + pu[1]) + (pu[2] + pu[3])) + ((pu[4] + pu[5]) + (pu[6] + pu[7]))
                        : 0.0f;
          }
#pragma unroll
          for (int j = jg; j < jg + JG; ++j) {
            float lo, hi;
            rows16(s2[j], lo, hi);
            const float s1 = lo + hi;
            rows32(s1, lo, hi);
            s2[j] = lo + hi;
            if constexpr (EX == 2) {
              rows16(u2[j], lo, hi);
              const float u1 = lo + hi;
              rows32(u1, lo, hi);
              u2[j] = lo + hi;
            }
          }
        }
        // 3) tile-major [nST][T] statistics (coalesced over rows): row
        //    group 0 stores the max, 1 the sum, 2 the entropy partial, through
        //    buffer resources over this wave's 128 rows of the tile's row
        //    (rows past T lie past their size; the other row groups' lanes
        //    get an offset past it): no branch and no per-lane pointer.
        {
          constexpr uint32_t DROP = 0x80000000u;
          const int r0 = t0 + wt * WT;
          const size_t base = (size_t)(a.js_base + js) * a.T + r0;
          const uint32_t bytes = r0 < a.T ? (uint32_t)min(WT, a.T - r0) * 4u : 0u;
          const __amdgpu_buffer_rsrc_t r_m = make_rsrc(a.part_m + base, bytes);
          const __amdgpu_buffer_rsrc_t r_s = make_rsrc(a.part_s + base, bytes);
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            const uint32_t off = (uint32_t)(16 * j + fc) * 4u;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m2[j]), r_m,
                                                  (int)(fg == 0 ? off : DROP), 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s2[j]), r_s,
                                                  (int)(fg == 1 ? off : DROP), 0, 0);
          }
          if constexpr (EX == 2) {
            const __amdgpu_buffer_rsrc_t r_u = make_rsrc(a.part_u + base, bytes);
#pragma unroll
            for (int j = 0; j < NJ; ++j)
              __builtin_amdgcn_raw_buffer_store_b32(
                  __float_as_uint(u2[j]), r_u,
                  (int)(fg == 2 ? (uint32_t)(16 * j + fc) * 4u : DROP), 0, 0);
          }
        }
        // 4) target capture: the one lane holding z[t][y[t]] writes xt[t],
        //    the value picked by a fixed select tree over its 32 values.
        // (targets are global ids; a weight slice starts at y_base)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int t = t0 + wt * WT + 16 * j + fc;
          const int yt = target_of(j, t);
          const int y = yt < 0 ? -1 : yt - a.y_base;
          const int rel = y - vbase;
          const bool hit = rel >= 0 && rel < STAT_V && ((rel >> 2) & 3) == fg;
          if (__any(hit)) {
            const float zy = pick(j, rel);
            if (hit) a.xt[t] = xf(zy);
          }
        }
      };
      // The vocabulary-tail column (V not a multiple of TILE_V) masks the
      // columns past V; the choice depends on the tile's column, i.e. on V.
      if (js < a.nST) {
        if (n == a.nVT - 1 && a.V % TILE_V != 0) stats_epilogue(std::true_type{});
        else stats_epilogue(std::false_type{});
      }
      }  // EX != 3
    }

    }  // epilogue scope
    if (!more_tiles) {
      // nothing of this wave's may still be writing LDS when it ends
      __builtin_amdgcn_s_waitcnt(VMCNT0);
      break;
    }
    parity ^= 1;
    L = Ln;
    m = mn;
    n = nn;
    rw = rsrc_w(n);
    rh = rsrc_h(m);
    pw = pf_rsrc(m, rw);
    ph = pfh_rsrc(rh);
  }
}

// Launch shapes: the statistics kernel is persistent (one workgroup per
// compute unit walking the tiles); the logits-stage kernel uses one
// workgroup per tile.
template <bool STATS, bool PERSIST, int EX, bool KMW>
__global__ __launch_bounds__(GEMM_THREADS) void gemm_kernel(const GemmArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[CLAIM_OFS + 16];
  gemm_body<STATS, PERSIST, EX, KMW>(a, smem);
}

// Per row t: M = max_j m_j (exact in any order), then
// s = sum_j s_j exp(m_j - M) as MERGE_GROUPS sequential folds over contiguous
// groups of ceil(nST / MERGE_GROUPS) statistics tiles, then the group sums
// folded in order 0 .. MERGE_GROUPS-1.  The shape depends only on nST.
// Slots past the group's end contribute max(-inf) and + 0 * exp(-inf) = + 0,
// which changes nothing (the running sum is never -0).
//
// With ENT, the same fold also carries U = sum_j e_j (u_j + (m_j - M) s_j),
// e_j = exp(m_j - M): the sum over the row of exp(z - M) (z - M), all terms
// <= 0, so H = log S - U / S involves no cancellation.
//
// A workgroup holds MERGE_ROWS = 32 rows x MERGE_GROUPS groups (a wave: 32
// consecutive rows of 2 groups, one 128-byte line per group and load), so a
// 4096-row batch spreads over 128 workgroups.  The time is the memory
// latency of each round of loads, so KEEP (groups of at most MERGE_KEEP
// tiles, every vocabulary up to 163 840 entries) issues all of a group's
// loads at once and keeps the values in registers for both passes: one
// round trip.  Otherwise the statistics are read in chunks of MERGE_UNROLL,
// twice.  Both paths fold the same values in the same order.  (Measured,
// bitwise identical across layouts: 32 rows with KEEP 10.8 / 29.3 us at
// 4096 / 16384 rows, against 16 rows 14.7 / 50.3 us and 64 rows in chunks
// 16.2 / 35.2 us.)
template <bool ENT, bool KEEP>
__global__ __launch_bounds__(MERGE_GROUPS * MERGE_ROWS) void merge_kernel(
    const MergeArgs a) {
  __shared__ float red[MERGE_GROUPS][MERGE_ROWS];
  __shared__ float redu[ENT ? MERGE_GROUPS : 1][MERGE_ROWS];
  const int lane = threadIdx.x % MERGE_ROWS;
  const int g = threadIdx.x / MERGE_ROWS;
  const int t = blockIdx.x * MERGE_ROWS + lane;
  const bool valid = t < a.T;
  const int gs = (a.nST + MERGE_GROUPS - 1) / MERGE_GROUPS;
  const int j0 = min(a.nST, g * gs);
  const int j1 = min(a.nST, j0 + gs);
  const size_t T = (size_t)a.T;
  const float *pm = a.part_m + (valid ? t : 0) + (size_t)j0 * T;
  const float *ps = a.part_s + (valid ? t : 0) + (size_t)j0 * T;
  const float *pu = ENT ? a.part_u + (valid ? t : 0) + (size_t)j0 * T : nullptr;
  const int cnt = valid ? j1 - j0 : 0;   // tiles of this group

  constexpr int C = KEEP ? MERGE_KEEP : MERGE_UNROLL;
  float vm[C], vs[C], vu[ENT ? C : 1];
  auto load = [&](int base, bool with_m, bool with_su) {
#pragma unroll
    for (int u = 0; u < C; ++u) {
      const bool in = base + u < cnt;
      const size_t o = (size_t)(base + u) * T;
      if (with_m) vm[u] = in ? pm[o] : -INFINITY;
      if (with_su) {
        vs[u] = in ? ps[o] : 0.0f;
        if constexpr (ENT) vu[u] = in ? pu[o] : 0.0f;
      }
    }
  };

  float mg = -INFINITY;
  if constexpr (KEEP) load(0, true, true);
  for (int b = 0; b < (KEEP ? 1 : cnt); b += C) {
    if constexpr (!KEEP) load(b, true, false);
#pragma unroll
    for (int u = 0; u < C; ++u) mg = fmaxf(mg, vm[u]);
  }
  red[g][lane] = mg;
  __syncthreads();
  float M = red[0][lane];
#pragma unroll
  for (int q = 1; q < MERGE_GROUPS; ++q) M = fmaxf(M, red[q][lane]);
  __syncthreads();
  const float Ms = (M == -INFINITY) ? 0.0f : M;

  float sg = 0.0f, ug = 0.0f;
  for (int b = 0; b < (KEEP ? 1 : cnt); b += C) {
    if constexpr (!KEEP) load(b, true, true);
#pragma unroll
    for (int u = 0; u < C; ++u) {
      const float dm = vm[u] - Ms;
      const float e = __builtin_amdgcn_exp2f(dm * LOG2E);
      sg = sg + vs[u] * e;
      // a tile with m_j = -inf has s_j = u_j = 0 and e = 0: it adds 0
      if constexpr (ENT) ug = ug + e * (vu[u] + fmaxf(dm, -FLT_MAX) * vs[u]);
    }
  }
  red[g][lane] = sg;
  if constexpr (ENT) redu[g][lane] = ug;
  __syncthreads();
  if (g == 0 && valid) {
    float sum = red[0][lane];
#pragma unroll
    for (int q = 1; q < MERGE_GROUPS; ++q) sum = sum + red[q][lane];
    const float logs = __builtin_amdgcn_logf(sum) * LN2;
    const float lse = M + logs;
    const int y = a.targets[t];
    a.lse[t] = lse;
    a.logp[t] = (y >= 0 && y < a.V) ? a.xt[t] - lse : __builtin_nanf("");
    if constexpr (ENT) {
      float us = redu[0][lane];
#pragma unroll
      for (int q = 1; q < MERGE_GROUPS; ++q) us = us + redu[q][lane];
      // a row whose lse is not finite has no entropy
      a.entropy[t] = (lse == lse && fabsf(lse) != INFINITY) ? logs - us / sum
                                                            : __builtin_nanf("");
    }
  }
}

__global__ __launch_bounds__(COMPARE_THREADS) void compare_kernel(
    const float *__restrict__ x, const float *__restrict__ y, int64_t n,
    double *__restrict__ stats) {
  __shared__ double sd[4][COMPARE_THREADS];
  __shared__ long long sc[2][COMPARE_THREADS];
  const int tid = threadIdx.x;
  long long mism = 0, kcnt = 0;
  double mx = 0.0, sa = 0.0, sq = 0.0, k3 = 0.0;
  // Elements tid, tid + COMPARE_THREADS, ... in increasing order; the loads
  // of COMPARE_UNROLL of them are issued together (one memory round trip per
  // 4096 elements instead of one per element a thread visits).
  // element indices in 64 bits: n may come within a stride of 2^31
  for (int64_t base = 0; base < n; base += COMPARE_THREADS * COMPARE_UNROLL) {
    float xa[COMPARE_UNROLL], ya[COMPARE_UNROLL];
#pragma unroll
    for (int u = 0; u < COMPARE_UNROLL; ++u) {
      const int64_t i = base + u * COMPARE_THREADS + tid;
      xa[u] = i < n ? x[i] : 0.0f;
      ya[u] = i < n ? y[i] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < COMPARE_UNROLL; ++u) {
      if (base + u * COMPARE_THREADS + tid >= n) break;
      const float a = xa[u], b = ya[u];
      if (__float_as_uint(a) != __float_as_uint(b)) {
        ++mism;
        double d = fabs((double)a - (double)b);
        if (isnan(d)) d = INFINITY;
        mx = fmax(mx, d);
        sa = sa + d;
        sq = sq + d * d;
      }
      if (isfinite(a) && isfinite(b)) {
        // equal bits give lr = 0 and k3 = exp(0) - 1 - 0 = 0 exactly
        if (__float_as_uint(a) != __float_as_uint(b)) {
          const double lr = (double)a - (double)b;
          k3 = k3 + ((exp(lr) - 1.0) - lr);
        }
        ++kcnt;
      }
    }
  }
  sc[0][tid] = mism;
  sc[1][tid] = kcnt;
  sd[0][tid] = mx;
  sd[1][tid] = sa;
  sd[2][tid] = sq;
  sd[3][tid] = k3;
  __syncthreads();
  for (int s = COMPARE_THREADS / 2; s > 0; s >>= 1) {
    if (tid < s) {
      sc[0][tid] += sc[0][tid + s];
      sc[1][tid] += sc[1][tid + s];
      sd[0][tid] = fmax(sd[0][tid], sd[0][tid + s]);
      sd[1][tid] = sd[1][tid] + sd[1][tid + s];
      sd[2][tid] = sd[2][tid] + sd[2][tid + s];
      sd[3][tid] = sd[3][tid] + sd[3][tid + s];
    }
    __syncthreads();
  }
  if (tid == 0) {
    stats[0] = (double)n;
    stats[1] = (double)sc[0][0];
    stats[2] = sd[0][0];
    stats[3] = sd[1][0];
    stats[4] = sd[2][0];
    stats[5] = sd[3][0];
    stats[6] = (double)sc[1][0];
    stats[7] = 0.0;
  }
}

__global__ __launch_bounds__(256) void zero_kernel(float *x, int64_t n);

namespace {

// As few workgroups (a multiple of 8, so each stays on one XCD) as give the
// same number of rounds: a last round of a few workgroups, each waiting on
// its own weight stream, costs as much as a full one, while fewer concurrent
// workgroups share the bandwidth of every round (594 tiles of a decode batch:
// 200 workgroups x 3 rounds instead of 256 and a third round of 82).
int balanced_grid(int tiles, int workers) {
  int grid = workers >= 8 ? workers - workers % 8 : 8;
  if (grid > tiles) grid = tiles;
  if (grid % 8 == 0) {
    const int rounds = ceil_div(tiles, grid);
    grid = (ceil_div(tiles, rounds) + 7) / 8 * 8;
  }
  return grid;
}

template <int EX>
void launch_stats_kernel(const GemmArgs &a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((gemm_kernel<true, true, EX, false>), dim3(grid), dim3(GEMM_THREADS), 0, s,
                     a);
}

template <int EX>
void launch_store_kernel(const GemmArgs &a, int grid, hipStream_t s) {
  if constexpr (EX == 2) {   // transposed output: K-major weight role only
    hipLaunchKernelGGL((gemm_kernel<false, true, 2, true>), dim3(grid), dim3(GEMM_THREADS), 0,
                       s, a);
  } else {
    if (a.kmw)   // the weight-role operand K-major (the product over the vocabulary)
      hipLaunchKernelGGL((gemm_kernel<false, true, EX, true>), dim3(grid), dim3(GEMM_THREADS),
                         0, s, a);
    else
      hipLaunchKernelGGL((gemm_kernel<false, true, EX, false>), dim3(grid), dim3(GEMM_THREADS),
                         0, s, a);
  }
}

}  // namespace

// Every batch size runs the one 256 x 256 tile; only the number of
// workgroups of the persistent walk (the schedule) depends on the tile count.
hipError_t launch_gemm_stats(const GemmArgs &a, int workers, hipStream_t s) {
  const int grid = balanced_grid(a.nMT * a.nVT, workers);
  // the claim counters start at zero (a kernel, not a memset: capturable)
  if (a.queue) hipLaunchKernelGGL(zero_kernel, dim3(1), dim3(64), 0, s, (float *)a.queue, 8);
  if (a.ex == 3) launch_stats_kernel<3>(a, grid, s);
  else if (a.ex == 2) launch_stats_kernel<2>(a, grid, s);
  else if (a.ex == 1) launch_stats_kernel<1>(a, grid, s);
  else launch_stats_kernel<0>(a, grid, s);
  return hipGetLastError();
}

hipError_t launch_gemm_logits(const GemmArgs &a, int workers, hipStream_t s) {
  const int grid = balanced_grid(a.nMT * a.nVT, workers);
  if (a.queue) hipLaunchKernelGGL(zero_kernel, dim3(1), dim3(64), 0, s, (float *)a.queue, 8);
  // whole rows through LDS when V is a multiple of 4 and the output 16-byte
  // aligned; otherwise one column per store (the same values)
  const bool vec = (a.V & 3) == 0 && ((uintptr_t)a.logits & 15) == 0;
  if (a.out_t) {
    // transposed: whole 16-byte pieces of rows of T columns (T % 4 == 0)
    if (!a.kmw || (a.T & 3) != 0 || ((uintptr_t)a.logits & 15) != 0)
      return hipErrorInvalidValue;
    launch_store_kernel<2>(a, grid, s);
  } else if (vec) launch_store_kernel<0>(a, grid, s);
  else launch_store_kernel<1>(a, grid, s);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs &a, hipStream_t s) {
  const dim3 grid(ceil_div(a.T, MERGE_ROWS)), block(MERGE_GROUPS * MERGE_ROWS);
  // which path depends only on the vocabulary size; both give the same bits
  const bool keep = ceil_div(a.nST, MERGE_GROUPS) <= MERGE_KEEP;
  if (a.entropy) {
    if (keep) hipLaunchKernelGGL((merge_kernel<true, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((merge_kernel<true, false>), grid, block, 0, s, a);
  } else {
    if (keep) hipLaunchKernelGGL((merge_kernel<false, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((merge_kernel<false, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

// 64 x 64 tiles through LDS, moved as 16-byte chunks of 8 elements: a
// thread reads 8 consecutive columns of one input row and writes 8
// consecutive columns (input rows) of one output row.  Requires C % 64 == 0,
// ldi % 8 == 0 and ldo % 64 == 0 (checked by the caller).
constexpr int TR_TILE = 64;
constexpr int TR_PITCH = TR_TILE + 8;   // LDS row pitch in elements (16-byte aligned)
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t *__restrict__ in,
                                                        int64_t ldi, int R, int C,
                                                        uint16_t *__restrict__ out,
                                                        int64_t ldo) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[TR_TILE][TR_PITCH];
  const int r0 = blockIdx.x * TR_TILE;   // output columns (the long side) in x
  const int c0 = blockIdx.y * TR_TILE;
  const int chunk = threadIdx.x & 7, y0 = threadIdx.x >> 3;   // 32 rows x 8 chunks
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int rr = y0 + 32 * pass;
    const int r = r0 + rr;
    uint4 x = make_uint4(0, 0, 0, 0);
    if (r < R) x = *(const uint4 *)(in + (size_t)r * ldi + c0 + 8 * chunk);
    *(uint4 *)&tile[rr][8 * chunk] = x;
  }
  __syncthreads();
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int cc = y0 + 32 * pass;       // output row c0 + cc
    uint16_t e[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) e[k] = tile[8 * chunk + k][cc];
    uint4 x;
    x.x = e[0] | ((uint32_t)e[1] << 16);
    x.y = e[2] | ((uint32_t)e[3] << 16);
    x.z = e[4] | ((uint32_t)e[5] << 16);
    x.w = e[6] | ((uint32_t)e[7] << 16);
    if (r0 + 8 * chunk < ldo) *(uint4 *)(out + (size_t)(c0 + cc) * ldo + r0 + 8 * chunk) = x;
  }
}

hipError_t launch_transpose(const uint16_t *in, int64_t ldi, int R, int C, uint16_t *out,
                            int64_t ldo, hipStream_t s) {
  hipLaunchKernelGGL(transpose_kernel, dim3(ceil_div(ldo, TR_TILE), ceil_div(C, TR_TILE)),
                     dim3(256), 0, s, in, ldi, R, C, out, ldo);
  return hipGetLastError();
}

// RMSNorm, one wave per row, RMS_ROWS rows per workgroup.  Lane l owns the
// 16-byte chunks l, l + 64, l + 128, ... of the row; it sums their squares in
// element order, then the lanes combine in a butterfly (xor 32, 16, .., 1):
// partners add the same two numbers, so every lane ends with the same total,
// whose association depends only on H.  r = 1 / sqrt(ss / H + eps) with IEEE
// square root and division; y = bf16(bf16(x r) gamma), where the second
// product, of two bf16 values, is exact in fp32.
constexpr int RMS_ROWS = 4;
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// NC > 0: the row has at most NC chunks per lane (H <= 512 NC); all of them,
// and gamma's, are loaded at once and the row is kept in registers (one
// memory round trip).  NC == 0: any H, the row read twice (the second time
// from L2).  Same arithmetic, same order.
template <int NC>
__global__ __launch_bounds__(64 * RMS_ROWS) void rmsnorm_kernel(
    const uint16_t *__restrict__ x, int64_t ldx, const uint16_t *__restrict__ gamma, float eps,
    uint16_t *__restrict__ y, int64_t ldy, int T, int H) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * RMS_ROWS + (threadIdx.x >> 6);
  if (t >= T) return;                      // a whole wave
  const uint16_t *row = x + (size_t)t * ldx;
  uint16_t *out = y + (size_t)t * ldy;
  const int nch = H >> 3;
  auto sum_sq = [](float ss, const uint4 &v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float a = bf16_lo(w[k]), b = bf16_hi(w[k]);
      ss = ss + a * a;
      ss = ss + b * b;
    }
    return ss;
  };
  auto norm = [](const uint4 &v, const uint4 &g, float r) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    const uint32_t gw[4] = {g.x, g.y, g.z, g.w};
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float n0 = bf16_lo(bf16_bits(bf16_lo(w[k]) * r));
      const float n1 = bf16_lo(bf16_bits(bf16_hi(w[k]) * r));
      o[k] = bf16_bits(n0 * bf16_lo(gw[k])) | (bf16_bits(n1 * bf16_hi(gw[k])) << 16);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
  };
  float ss = 0.0f;
  if constexpr (NC > 0) {
    uint4 v[NC], g[NC];
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      const int c = lane + 64 * u;
      v[u] = make_uint4(0, 0, 0, 0);
      g[u] = make_uint4(0, 0, 0, 0);
      if (c < nch) {
        v[u] = *(const uint4 *)(row + 8 * c);
        g[u] = *(const uint4 *)(gamma + 8 * c);
      }
    }
#pragma unroll
    for (int u = 0; u < NC; ++u)
      if (lane + 64 * u < nch) ss = sum_sq(ss, v[u]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ss = ss + __shfl_xor(ss, o);
    const float r = 1.0f / sqrtf(ss / (float)H + eps);
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      const int c = lane + 64 * u;
      if (c < nch) *(uint4 *)(out + 8 * c) = norm(v[u], g[u], r);
    }
  } else {
    for (int c = lane; c < nch; c += 64) ss = sum_sq(ss, *(const uint4 *)(row + 8 * c));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ss = ss + __shfl_xor(ss, o);
    const float r = 1.0f / sqrtf(ss / (float)H + eps);
    for (int c = lane; c < nch; c += 64)
      *(uint4 *)(out + 8 * c) =
          norm(*(const uint4 *)(row + 8 * c), *(const uint4 *)(gamma + 8 * c), r);
  }
}

hipError_t launch_rmsnorm(const uint16_t *x, int64_t ldx, const uint16_t *gamma, float eps,
                          uint16_t *y, int64_t ldy, int T, int H, hipStream_t s) {
  const dim3 grid(ceil_div(T, RMS_ROWS)), block(64 * RMS_ROWS);
  // the smallest register-resident instantiation that holds the row (the
  // choice depends only on H; all three compute the same bits)
  if (H <= 512 * 8)
    hipLaunchKernelGGL(rmsnorm_kernel<8>, grid, block, 0, s, x, ldx, gamma, eps, y, ldy, T, H);
  else if (H <= 512 * 16)
    hipLaunchKernelGGL(rmsnorm_kernel<16>, grid, block, 0, s, x, ldx, gamma, eps, y, ldy, T, H);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<0>, grid, block, 0, s, x, ldx, gamma, eps, y, ldy, T, H);
  return hipGetLastError();
}

// Top-k of one row per workgroup under the order (value descending, id
// ascending), a total order on (value, id) pairs, so the selection does not
// depend on the order candidates are visited or combined in.  Values are
// z' = z inv_tau (then rounded to bf16 if asked), exactly as the statistics
// kernel forms them, and logp = z' - lse as the merge does; NaN entries are
// never selected; missing entries (fewer than k non-NaN) get id -1, -inf.
//
// The statistics pass already holds every 128-wide tile's maximum of z'.
// If m* is the k-th largest of a row's tile maxima, the k tiles with the
// largest maxima hold k distinct entries >= m*, so the k-th largest entry is
// >= m*, and no tile whose maximum is below m* can hold a top-k entry.  So:
//   1) m* by a top-k selection over the row's tile maxima;
//   2) the list of tiles with maximum >= m* (more than TOPK_LIST of them,
//      possible only with ties, e.g. constant rows: scan the whole row);
//   3) a top-k selection over those tiles' entries: each thread keeps its
//      best k (unsorted, current minimum tracked), then k rounds of a
//      block-wide maximum in which the owner drops the winner.
constexpr int TOPK_THREADS = 256;
constexpr int TOPK_CPT = 32;   // candidates per thread held in registers (bisection path)
constexpr int TOPK_MPT = 8;    // tile maxima per thread held in registers (bisection path)
// Smallest k that takes the bisection path (k = 16 / 20, 4096 rows: rounds
// 0.25 / 0.47 ms, bisection 0.33 / 0.33 ms).
constexpr int TOPK_BISECT_K = 17;
constexpr int TOPK_LIST = 512;
struct Cand {
  float v;
  int i;
};
__device__ __forceinline__ bool cand_gt(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}
// Order-preserving key of a non-NaN float (larger value, larger key), with -0
// and +0 equal, as they are under cand_gt.
__device__ __forceinline__ uint32_t order_key(float z) {
  const uint32_t u = __float_as_uint(z == 0.0f ? 0.0f : z);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
template <int KC>
struct TopK {
  static constexpr int NONE = 0x7FFFFFFF;   // id of an empty slot: below every entry
  float val[KC];
  int idx[KC];
  float mval;
  int midx, mpos;
  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int q = 0; q < KC; ++q) {
      val[q] = -INFINITY;
      idx[q] = NONE;
    }
    mval = -INFINITY;
    midx = NONE;
    mpos = 0;
  }
  __device__ __forceinline__ void offer(float z, int v, int k) {
    if (!(z == z) || !cand_gt(z, v, mval, midx)) return;     // NaN, or not better
    // unconditional selects keep the slots in registers
#pragma unroll
    for (int q = 0; q < KC; ++q) {
      const bool hit = q == mpos;
      val[q] = hit ? z : val[q];
      idx[q] = hit ? v : idx[q];
    }
    mval = val[0];
    midx = idx[0];
    mpos = 0;
#pragma unroll
    for (int q = 1; q < KC; ++q)
      if (q < k && cand_gt(mval, midx, val[q], idx[q])) {
        mval = val[q];
        midx = idx[q];
        mpos = q;
      }
  }
  // Round r of the block-wide selection: the winner of the remaining
  // candidates, dropped by its owner, returned to every thread.
  __device__ __forceinline__ Cand next(int k, Cand *red, Cand *win) {
    const int tid = threadIdx.x;
    float bv = -INFINITY;
    int bi = NONE;
#pragma unroll
    for (int q = 0; q < KC; ++q)
      if (q < k && cand_gt(val[q], idx[q], bv, bi)) {
        bv = val[q];
        bi = idx[q];
      }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o);
      const int oi = __shfl_xor(bi, o);
      if (cand_gt(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((tid & 63) == 0) red[tid >> 6] = Cand{bv, bi};
    __syncthreads();
    if (tid == 0) {
      Cand w = red[0];
#pragma unroll
      for (int q = 1; q < TOPK_THREADS / 64; ++q)
        if (cand_gt(red[q].v, red[q].i, w.v, w.i)) w = red[q];
      *win = w;
    }
    __syncthreads();
    const Cand w = *win;
    __syncthreads();   // every thread has read *win before the next round writes it
#pragma unroll
    for (int q = 0; q < KC; ++q) {
      const bool hit = idx[q] == w.i && w.i != NONE;
      val[q] = hit ? -INFINITY : val[q];
      idx[q] = hit ? NONE : idx[q];
    }
    return w;
  }
};

// A count summed over the workgroup of TOPK_THREADS threads (every thread
// gets the total); csum holds one slot per wave.
__device__ __forceinline__ int block_sum(int c, int *csum) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
  if ((threadIdx.x & 63) == 0) csum[threadIdx.x >> 6] = c;
  __syncthreads();
  int total = 0;
#pragma unroll
  for (int q = 0; q < TOPK_THREADS / 64; ++q) total += csum[q];
  __syncthreads();
  return total;
}

// m* of row t: the k-th largest of its tile maxima part_m[j][t] (the entries
// of this selection are the tiles), -inf when fewer than k tile maxima are
// not NaN.  Large k: by bisection on the order-preserving key (32 block-wide
// counts) instead of k rounds of a block-wide maximum; small k keep the
// rounds, which cost less there (the instantiations for k <= 16 carry no
// bisection code, for their registers).
template <int KC>
__device__ float kth_tile_max(const float *__restrict__ part_m, int t, int T, int nST, int k,
                              TopK<KC> &sel, Cand *red, Cand *win, int *csum) {
  const int tid = threadIdx.x;
  const bool bisect = KC >= 32 && k >= TOPK_BISECT_K;
  float mstar;
  if (KC >= 32 && bisect && nST <= TOPK_THREADS * TOPK_MPT) {
    uint32_t key[TOPK_MPT];
    bool ok[TOPK_MPT];
#pragma unroll
    for (int u = 0; u < TOPK_MPT; ++u) {
      const int j = u * TOPK_THREADS + tid;
      const float m = j < nST ? part_m[(size_t)j * T + t] : __builtin_nanf("");
      ok[u] = m == m;
      key[u] = order_key(m);
    }
    auto count_ge = [&](uint32_t kmin) {
      int c = 0;
#pragma unroll
      for (int u = 0; u < TOPK_MPT; ++u) c += (ok[u] && key[u] >= kmin) ? 1 : 0;
      return block_sum(c, csum);
    };
    if (count_ge(0) < k) {
      mstar = -INFINITY;
    } else {
      uint32_t K = 0;   // the largest key with at least k tile maxima at or above it
      for (int bit = 31; bit >= 0; --bit)
        if (count_ge(K | (1u << bit)) >= k) K |= 1u << bit;
      mstar = __uint_as_float((K & 0x80000000u) ? (K & 0x7FFFFFFFu) : ~K);
    }
  } else {
    sel.reset();
    for (int j = tid; j < nST; j += TOPK_THREADS) sel.offer(part_m[(size_t)j * T + t], j, k);
    Cand kth{-INFINITY, TopK<KC>::NONE};
    const int kk = k < nST ? k : nST;
    for (int r = 0; r < kk; ++r) kth = sel.next(k, red, win);
    mstar = kth.v;
  }
  return mstar;
}

// The candidate-pair source of the selection (rlk_topk_logp_direct): row
// t's candidates are the tiles cand_tile[t C + u], u < cand_n[t], whose 128
// raw logits sit at pair t C + u of pair_z (128 floats per pair).
// cand_n[t] < 0 marks a row whose k-th largest tile maximum is -inf: all its
// tiles are candidates, tile j at pair t C + j when nST <= C, else at pair
// T C + d nST + j with d = deg_rank[t] (d < 0: the workspace had no room
// for the row).
struct PairSrc {
  const int *cand_n;
  const int *cand_tile;
  const int *deg_rank;
  const float *pair_z;
  int C;
  int all_tiles_only;   // skip the rows with k candidate tiles (a wave per row took them)
};

template <int KC, bool PAIRS>
__global__ __launch_bounds__(TOPK_THREADS) void topk_kernel(
    const float *__restrict__ logits, int64_t ld, const float *__restrict__ lse,
    const float *__restrict__ part_m, int T, int V, int nST, int k, float inv_tau, int bf16,
    float *__restrict__ out_lp, int32_t *__restrict__ out_id, const PairSrc ps) {
  __shared__ Cand red[TOPK_THREADS / 64];
  __shared__ Cand win;
  __shared__ int list[TOPK_LIST];
  __shared__ int nlist;
  __shared__ int csum[TOPK_THREADS / 64];
  __shared__ float win_v[64];
  __shared__ int win_i[64];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const float *row = PAIRS ? nullptr : logits + (size_t)t * ld;
  TopK<KC> sel;
  const bool bisect = KC >= 32 && k >= TOPK_BISECT_K;

  float mstar = 0.0f;
  int n;
  int64_t dbase = 0;   // pairs, whole row: tile j's logits are at pair dbase + j
  if constexpr (PAIRS) {
    const int cn = ps.cand_n[t];
    if (cn >= 0 && ps.all_tiles_only) return;
    if (cn >= 0) {
      for (int u = tid; u < cn; u += TOPK_THREADS) list[u] = ps.cand_tile[(size_t)t * ps.C + u];
      n = cn;
    } else {
      if (nST <= ps.C) {
        dbase = (int64_t)t * ps.C;
      } else {
        const int d = ps.deg_rank[t];
        if (d < 0) {   // no room for this row's tiles: marked, not guessed
          if (tid < k) {
            out_lp[(size_t)t * k + tid] = __builtin_nanf("");
            out_id[(size_t)t * k + tid] = -2;
          }
          return;
        }
        dbase = (int64_t)T * ps.C + (int64_t)d * nST;
      }
      n = TOPK_LIST + 1;   // the whole row
    }
    __syncthreads();
  } else {
    // 1) m*: the k-th largest tile maximum
    mstar = kth_tile_max<KC>(part_m, t, T, nST, k, sel, red, &win, csum);
    // 2) the tiles that can hold a top-k entry
    if (tid == 0) nlist = 0;
    __syncthreads();
    for (int j = tid; j < nST; j += TOPK_THREADS) {
      const float m = part_m[(size_t)j * T + t];
      if (m >= mstar) {
        const int at = atomicAdd(&nlist, 1);
        if (at < TOPK_LIST) list[at] = j;
      }
    }
    __syncthreads();
    n = nlist;
  }
  // raw logit of list candidate i (entry v), and of entry v of the whole row
  auto zl = [&](int i, int v) -> float {
    if constexpr (PAIRS)
      return ps.pair_z[((size_t)t * ps.C + i / STAT_V) * STAT_V + (i % STAT_V)];
    else
      return row[v];
  };
  auto zr = [&](int v) -> float {
    if constexpr (PAIRS)
      return ps.pair_z[(size_t)(dbase + v / STAT_V) * STAT_V + (v % STAT_V)];
    else
      return row[v];
  };

  // 3) top-k of those tiles' entries (or of the whole row)
  const float l = lse[t];
  if (KC >= 32 && bisect && n <= TOPK_LIST && mstar == mstar &&
      n * STAT_V <= TOPK_THREADS * TOPK_CPT) {
    // Up to TOPK_CPT candidates per thread, held in registers.  The k-th
    // largest value is found by bisection on its order-preserving key (32
    // block-wide counts), the ties at that key by bisection on the id (the
    // smallest ids win): exactly the entries the order (value descending, id
    // ascending) puts first, in O(32) rounds instead of k.  The winners are
    // then ranked against each other in LDS.
    const int ne = n * STAT_V;
    uint32_t key[TOPK_CPT];
    int cid[TOPK_CPT];
    float cz[TOPK_CPT];
#pragma unroll
    for (int u = 0; u < TOPK_CPT; ++u) {
      const int i = u * TOPK_THREADS + tid;
      const int v = i < ne ? list[i / STAT_V] * STAT_V + (i % STAT_V) : V;
      float z = v < V ? zl(i, v) : __builtin_nanf("");
      z = z * inv_tau;
      if (bf16) z = (float)(__bf16)z;
      cz[u] = z;
      cid[u] = v < V && z == z ? v : -1;            // -1: no candidate (past V, or NaN)
      key[u] = order_key(z);
    }
    auto count = [&](auto pred) {
      int c = 0;
#pragma unroll
      for (int u = 0; u < TOPK_CPT; ++u) c += (cid[u] >= 0 && pred(u)) ? 1 : 0;
      return block_sum(c, csum);
    };
    const int nvalid = count([](int) { return true; });
    const int kk = k < nvalid ? k : nvalid;
    uint32_t K = 0;   // the largest key with at least kk entries at or above it
    int x = 0;        // the largest id below which fewer than `need` ties lie
    if (kk > 0) {
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t trial = K | (1u << bit);
        if (count([&](int u) { return key[u] >= trial; }) >= kk) K = trial;
      }
      const int need = kk - count([&](int u) { return key[u] > K; });
      // ids are below V: bits 30 - clz(V - 1) .. 0 cover them (V <= 2^31 - 1)
      const int top = V > 1 ? 31 - __clz(V - 1) : 0;
      for (int bit = top; bit >= 0; --bit) {
        const int trial = x | (1 << bit);
        if (count([&](int u) { return key[u] == K && cid[u] < trial; }) < need) x = trial;
      }
    }
    if (tid == 0) nlist = 0;   // reused as the winner count
    __syncthreads();
#pragma unroll
    for (int u = 0; u < TOPK_CPT; ++u)
      if (cid[u] >= 0 && kk > 0 && (key[u] > K || (key[u] == K && cid[u] <= x))) {
        const int at = atomicAdd(&nlist, 1);
        win_v[at] = cz[u];
        win_i[at] = cid[u];
      }
    __syncthreads();
    if (tid < kk) {
      int rank = 0;
      for (int q = 0; q < kk; ++q) rank += cand_gt(win_v[q], win_i[q], win_v[tid], win_i[tid]);
      out_lp[(size_t)t * k + rank] = win_v[tid] - l;
      out_id[(size_t)t * k + rank] = win_i[tid];
    } else if (tid < k) {
      out_lp[(size_t)t * k + tid] = -INFINITY;
      out_id[(size_t)t * k + tid] = -1;
    }
    return;
  }
  sel.reset();
  auto offer_z = [&](float z, int v) {
    z = z * inv_tau;
    if (bf16) z = (float)(__bf16)z;
    sel.offer(z, v, k);
  };
  if (n <= TOPK_LIST && mstar == mstar) {
    for (int i = tid; i < n * STAT_V; i += TOPK_THREADS) {
      const int v = list[i / STAT_V] * STAT_V + (i % STAT_V);
      if (v < V) offer_z(zl(i, v), v);
    }
  } else {
    for (int v = tid; v < V; v += TOPK_THREADS) offer_z(zr(v), v);
  }
  for (int r = 0; r < k; ++r) {
    const Cand w = sel.next(k, red, &win);
    if (tid == 0) {
      out_lp[(size_t)t * k + r] = w.i == TopK<KC>::NONE ? -INFINITY : w.v - l;
      out_id[(size_t)t * k + r] = w.i == TopK<KC>::NONE ? -1 : w.i;
    }
  }
}

hipError_t launch_topk(const float *logits, int64_t ld, const float *lse, const float *part_m,
                       int T, int V, int k, float inv_tau, int bf16, float *out_lp,
                       int32_t *out_id, hipStream_t s) {
  const int nST = ceil_div(V, STAT_V);
  if (k <= 8)
    hipLaunchKernelGGL((topk_kernel<8, false>), dim3(T), dim3(TOPK_THREADS), 0, s, logits, ld, lse, part_m,
                       T, V, nST, k, inv_tau, bf16, out_lp, out_id, PairSrc{});
  else if (k <= 16)
    hipLaunchKernelGGL((topk_kernel<16, false>), dim3(T), dim3(TOPK_THREADS), 0, s, logits, ld, lse,
                       part_m, T, V, nST, k, inv_tau, bf16, out_lp, out_id, PairSrc{});
  else if (k <= 32)
    hipLaunchKernelGGL((topk_kernel<32, false>), dim3(T), dim3(TOPK_THREADS), 0, s, logits, ld, lse,
                       part_m, T, V, nST, k, inv_tau, bf16, out_lp, out_id, PairSrc{});
  else
    hipLaunchKernelGGL((topk_kernel<64, false>), dim3(T), dim3(TOPK_THREADS), 0, s, logits, ld, lse,
                       part_m, T, V, nST, k, inv_tau, bf16, out_lp, out_id, PairSrc{});
  return hipGetLastError();
}

// ------------------------------------------------ top-k from the operands
// rlk_topk_logp_direct: the top-k selection above, but the logits of the
// candidate tiles are recomputed instead of read from a stored [T][V]
// array.  Candidate tiles of row t (m* its k-th largest tile maximum):
//   A: the tiles whose maximum exceeds m* (fewer than k of them: the k-th
//      largest maximum is m*);
//   B: the first k - |A| tiles, by index, whose maximum equals m*.
// Every top-k entry lies in A or B.  Entries above m* lie in A.  The entries
// equal to m* that make the cut are the smallest ids among all entries equal
// to m*; each tile of B holds at least one (its maximum, a value of the row),
// so the first k - |A| of them hold at least k - |A| >= the number needed,
// and any tile of B past them holds only larger ids.  So a row has exactly
// k candidate tiles.  When m* is -inf (fewer than k tiles hold a value above
// -inf: rows of NaN or infinities) every tile is a candidate.
//
// The logits of a (row, tile) pair come from the same MFMA instruction over
// the same operands in the same K order as the logit GEMM (16 x 16 x 32 bf16,
// fp32 accumulator from 0, K steps of 32 in increasing order with the same K
// slice in each lane, and the zero block the GEMM appends when H / 64 is
// odd), so they are the GEMM's bits: the
// selection sees exactly the values the stored-logits path reads.

// 1) per row: m*, the candidate tiles into the row's k slots, and one count
//    per candidate on its tile.
template <int KC>
__global__ __launch_bounds__(TOPK_THREADS) void topk_cand_kernel(const TopkDirectArgs a) {
  __shared__ Cand red[TOPK_THREADS / 64];
  __shared__ Cand win;
  __shared__ int csum[TOPK_THREADS / 64];
  __shared__ int nA;
  const int t = blockIdx.x, tid = threadIdx.x;
  const int T = a.T, nST = a.nST, k = a.k, C = a.C;
  TopK<KC> sel;
  const float mstar = kth_tile_max<KC>(a.part_m, t, T, nST, k, sel, red, &win, csum);
  int *tiles = a.cand_tile + (size_t)t * C;
  const float *pm = a.part_m + t;   // column t of [nST][T]
  if (!(mstar > -INFINITY)) {
    // every tile; with nST <= C they use the row's own slots, otherwise the
    // plan assigns room (and counts them) in row order
    if (tid == 0) a.cand_n[t] = -1;
    if (nST <= C)
      for (int j = tid; j < nST; j += TOPK_THREADS) atomicAdd(&a.tile_count[j], 1);
    return;
  }
  if (tid == 0) nA = 0;
  __syncthreads();
  for (int j = tid; j < nST; j += TOPK_THREADS)
    if (pm[(size_t)j * T] > mstar) {
      const int at = atomicAdd(&nA, 1);
      tiles[at] = j;
      atomicAdd(&a.tile_count[j], 1);
    }
  __syncthreads();
  const int na = nA;
  const int need = k - na;
  const int lane = tid & 63, w = tid >> 6;
  int taken = 0;   // tied tiles met so far (uniform)
  for (int base = 0; base < nST && taken < need; base += TOPK_THREADS) {
    const int j = base + tid;
    const bool f = j < nST && pm[(size_t)j * T] == mstar;
    const uint64_t b = __ballot(f);
    const int before = __popcll(b & ((1ull << lane) - 1ull));
    if (lane == 0) csum[w] = __popcll(b);
    __syncthreads();
    int wbase = 0, total = 0;
#pragma unroll
    for (int q = 0; q < TOPK_THREADS / 64; ++q) {
      wbase += q < w ? csum[q] : 0;
      total += csum[q];
    }
    __syncthreads();
    const int r = taken + wbase + before;
    if (f && r < need) {
      tiles[na + r] = j;
      atomicAdd(&a.tile_count[j], 1);
    }
    taken += total;
  }
  if (tid == 0) a.cand_n[t] = na + (taken < need ? taken : need);
}

// 2) one workgroup: room for the rows with m* = -inf (the first dcap in row
//    order, when nST > C), then per tile its pair count, its first pair slot
//    and its work items (a.tl_pairs pairs each, in tile order), and the tile of every
//    work item.
constexpr int PLAN_THREADS = 1024;
__global__ __launch_bounds__(PLAN_THREADS) void topk_plan_kernel(const TopkDirectArgs a) {
  __shared__ int wsum[PLAN_THREADS / 64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // exclusive prefix of x over the workgroup; `total` gets the sum
  auto scan = [&](int x, int &total) {
    int incl = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    int wb = 0;
    total = 0;
#pragma unroll
    for (int q = 0; q < PLAN_THREADS / 64; ++q) {
      wb += q < w ? wsum[q] : 0;
      total += wsum[q];
    }
    __syncthreads();
    return wb + incl - x;
  };
  int served = 0;
  if (a.nST > a.C) {
    int running = 0;
    for (int base = 0; base < a.T; base += PLAN_THREADS) {
      const int t = base + tid;
      const int f = (t < a.T && a.cand_n[t] < 0) ? 1 : 0;
      int tot;
      const int r = running + scan(f, tot);
      if (f) {
        const int d = r < a.dcap ? r : -1;
        a.deg_rank[t] = d;
        if (d >= 0) a.deg_row[d] = t;
      }
      running += tot;
    }
    served = running < a.dcap ? running : a.dcap;
  }
  int carry_p = 0, carry_i = 0;
  for (int base = 0; base < a.nST; base += PLAN_THREADS) {
    const int j = base + tid;
    const int c = j < a.nST ? a.tile_count[j] + served : 0;
    int tp, ti;
    const int op = scan(c, tp);
    const int oi = scan((c + a.tl_pairs - 1) / a.tl_pairs, ti);
    if (j < a.nST) {
      a.tile_count[j] = c;
      a.tile_off[j] = carry_p + op;
      a.item_off[j] = carry_i + oi;
      a.tile_fill[j] = 0;
    }
    carry_p += tp;
    carry_i += ti;
  }
  if (tid == 0) {
    a.item_off[a.nST] = carry_i;
    a.totals[0] = carry_i;
    a.totals[1] = carry_p;
  }
  __syncthreads();
  for (int j = tid; j < a.nST; j += PLAN_THREADS)
    for (int it = a.item_off[j]; it < a.item_off[j + 1]; ++it) a.item_tile[it] = j;
}

// 3) per row: its pairs into their tiles' buckets (a pair's place inside its
//    bucket changes which work item computes it, never its bits).
__global__ __launch_bounds__(64) void topk_scatter_kernel(const TopkDirectArgs a) {
  const int t = blockIdx.x, l = threadIdx.x;
  const int cn = a.cand_n[t];
  auto put = [&](int j, int p) {
    a.bucket[a.tile_off[j] + atomicAdd(&a.tile_fill[j], 1)] = p;
  };
  if (cn >= 0) {
    for (int u = l; u < cn; u += 64) put(a.cand_tile[(size_t)t * a.C + u], t * a.C + u);
  } else if (a.nST <= a.C) {
    for (int j = l; j < a.nST; j += 64) put(j, t * a.C + j);
  } else {
    const int d = a.deg_rank[t];
    if (d >= 0)
      for (int j = l; j < a.nST; j += 64) put(j, a.T * a.C + d * a.nST + j);
  }
}

// 4) one workgroup of NW waves per work item: the 128 x (up to 32 NW) logits
//    of one tile for up to a.tl_pairs = 32 NW of its pairs, wave w taking
//    pairs 32 w .. 32 w + 31 (NW = 8 when k > 32: a tile then holds about
//    twice as many pairs, and one item streams its weights once).
//    The tile's weight block (128 rows x 64 K, 16 KiB) goes to LDS by
//    direct-to-LDS loads, double-buffered and shared by the waves, in the
//    logit GEMM's layout (16-byte chunk c of row r at c ^ swz(r); load q of
//    wave w fills rows 8 (NW q + w) .. + 7).  The wave's pairs are two
//    16-column MFMA blocks: lane l loads the hidden rows of its pairs
//    l & 15 and 16 + (l & 15) straight into the MFMA operand layout (K slice
//    8 (l >> 4) .. + 7 of each 32-deep step), one block ahead.  Every logit
//    is the logit GEMM's: the same MFMA instruction over the same 32-deep K
//    slices in the same order, with the same K slice in each lane.  Rows
//    past V read zeros through the resource's range.
typedef char TileStage[TILE_K * STAT_V * 2];
template <int NW>
__device__ __forceinline__ void tile_logits_body(const TopkDirectArgs &a, TileStage *wlds) {
  constexpr int LQ = 16 / NW;   // 1 KiB weight loads per wave and K block
  const int it = blockIdx.x;
  if (it >= a.totals[0]) return;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, c = l & 15, g = l >> 4;
  const int j = a.item_tile[it];
  const int first = a.tile_off[j] + 32 * NW * (it - a.item_off[j]) + 32 * wave;
  const int cnt = min(32, a.tile_off[j] + a.tile_count[j] - first);   // <= 0: an idle wave
  const int regular = a.T * a.C;
  // the lane's pairs in blocks 0 and 1 (p < 0: none; its column is not stored)
  int pj[2];
  const uint16_t *hp[2];
#pragma unroll
  for (int jb = 0; jb < 2; ++jb) {
    const int pc = 16 * jb + c;
    const int pp = pc < cnt ? a.bucket[first + pc] : -1;
    int t = -1;
    if (pp >= 0) t = pp < regular ? pp / a.C : a.deg_row[(pp - regular) / a.nST];
    pj[jb] = t >= 0 ? pp : -1;
    // (a lane without a pair loads row 0: the MFMA keeps each output column
    // to its own B column, and that column is not stored)
    hp[jb] = a.hidden + (size_t)(t >= 0 ? t : 0) * a.ldh + 8 * g;
  }
  const int v0 = j * STAT_V;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(
      a.weight + (size_t)v0 * a.ldw, (uint32_t)(min(STAT_V, a.V - v0) * a.ldw * 2));
  typedef __attribute__((address_space(3))) void lds_void;
  // load q of this wave: row 8 (NW q + wave) + (l >> 3), global chunk (l & 7) ^ swz(row)
  uint32_t gofs[LQ];
#pragma unroll
  for (int q = 0; q < LQ; ++q) {
    const int row = 8 * (NW * q + wave) + (l >> 3);
    gofs[q] = (uint32_t)(row * a.ldw * 2 + (((l & 7) ^ swz(row)) << 4));
  }
  auto wload = [&](int kb, int st) {
#pragma unroll
    for (int q = 0; q < LQ; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rw, (lds_void *)(&wlds[st][0] + (NW * q + wave) * 1024), 16, gofs[q],
          (uint32_t)kb * (TILE_K * 2), 0, 0);
  };

  // hidden fragments of a block: [K step][pair block]
  auto hload = [&](int kb, u32x4 (&hb)[2][2]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
        hb[ks][jb] = *(const u32x4 *)(hp[jb] + kb * TILE_K + 32 * ks);
  };
  f32x4 acc[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) acc[i][jb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const int nk = a.H / TILE_K;
  const bool live = cnt > 0;   // uniform per wave
  u32x4 hb0[2][2], hb1[2][2];
  auto mma = [&](int i, int jb, bf16x8 w8, bf16x8 h8) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[i][jb]) : "v"(w8), "v"(h8));
  };
  // K block kb from stage ST (== kb & 1); the next block's loads go to the
  // other stage and hidden-fragment set.  (MFMAs in inline assembly, as in
  // the logit GEMM; wait states after the zeroing and before the reads.)
  auto block = [&](int kb, auto stage) {
    constexpr int ST = decltype(stage)::value;
    u32x4(&cur)[2][2] = ST ? hb1 : hb0;
    u32x4(&nxt)[2][2] = ST ? hb0 : hb1;
    // this block's loads (every wave's) have landed; the other stage is free
    __builtin_amdgcn_s_waitcnt(VMCNT0);
    __syncthreads();
    if (kb + 1 < nk) {
      wload(kb + 1, ST ^ 1);
      if (live) hload(kb + 1, nxt);
    }
    if (live) {
      // the 16 weight fragments of the block (step ks, block i: x = 8 ks +
      // i) through a ring of four, each read three fragments ahead (more
      // registers would cost this LDS-bound kernel resident waves)
      bf16x8 w8[4];
      auto wread = [&](int x) {
        const int ks = x >> 3, row = 16 * (x & 7) + c;
        w8[x & 3] = *(const bf16x8 *)(&wlds[ST][0] + row * 128 + (((4 * ks + g) ^ swz(row)) << 4));
      };
#pragma unroll
      for (int x = 0; x < 3; ++x) wread(x);
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        if (x + 3 < 16) wread(x + 3);
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
          mma(x & 7, jb, w8[x & 3], __builtin_bit_cast(bf16x8, cur[x >> 3][jb]));
      }
    }
  };
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 4");
  __builtin_amdgcn_sched_barrier(0);
  wload(0, 0);
  if (live) hload(0, hb0);
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  int kb = 0;
  for (; kb + 1 < nk; kb += 2) {
    block(kb, S0{});
    block(kb + 1, S1{});
  }
  if (kb < nk) block(kb, S0{});
  if (!live) return;
  if (nk & 1) {
    // the GEMM's appended zero block: 2 steps of zero operands (the wait
    // states cover the zero operand's VALU write)
    const bf16x8 z = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
          asm volatile("s_nop 4\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %1, %0"
                       : "+a"(acc[i][jb])
                       : "v"(z));
  }
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
  __builtin_amdgcn_sched_barrier(0);
  // acc[i][jb][e] is the logit of column 16 i + 4 g + e of the tile for the
  // lane's pair of block jb; columns past V are stored as NaN, which no
  // selection takes
  const int lim = a.V - v0 - 4 * g;   // columns at offset < lim are entries
  const uint32_t qnan = 0x7FC00000u;
#pragma unroll
  for (int jb = 0; jb < 2; ++jb) {
    if (pj[jb] >= 0) {
      float *o = a.pair_z + (size_t)pj[jb] * STAT_V + 4 * g;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        u32x4 d;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          d[e] = 16 * i + e < lim ? __float_as_uint(acc[i][jb][e]) : qnan;
        *(u32x4 *)(o + 16 * i) = d;
      }
    }
  }
}

// The candidate step and the selection with one wave per row (rows with k
// candidate tiles; the tile maxima of a row or its k x 128 candidates held as
// order keys in registers): every count is a wave reduction, no workgroup
// barrier.  The same entries as the workgroup kernels, which remain for
// vocabularies of more than 64 x CW_MPL tiles (candidate step) and for the
// rows that need all their tiles (selection).
__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}
constexpr int CW_MPL = 32;   // tile maxima per lane: up to 2048 tiles

__global__ __launch_bounds__(256) void topk_cand_wave_kernel(const TopkDirectArgs a) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= a.T) return;   // the whole wave
  const int T = a.T, nST = a.nST, k = a.k, C = a.C;
  const float *pm = a.part_m + t;
  // tile j = 64 u + lane; key 0 marks no tile (past nST; a NaN maximum)
  uint32_t key[CW_MPL];
#pragma unroll
  for (int u = 0; u < CW_MPL; ++u) {
    const int j = 64 * u + lane;
    const float m = j < nST ? pm[(size_t)j * T] : __builtin_nanf("");
    key[u] = m == m ? order_key(m) : 0u;
  }
  // a count over the wave: per u the compare's lane mask, counted in the
  // scalar unit (no cross-lane reduction)
  auto count_ge = [&](uint32_t kmin) {   // kmin >= 1
    int c = 0;
#pragma unroll
    for (int u = 0; u < CW_MPL; ++u) c += __popcll(__ballot(key[u] >= kmin));
    return c;
  };
  uint32_t K = 0;   // the key of m*: the largest with at least k tile maxima at or above it
  if (count_ge(1u) >= k)
    for (int bit = 31; bit >= 0; --bit)
      if (count_ge(K | (1u << bit)) >= k) K |= 1u << bit;
  if (K == 0u || !(key_value(K) > -INFINITY)) {   // m* = -inf: every tile
    if (lane == 0) a.cand_n[t] = -1;
    if (nST <= C)
      for (int j = lane; j < nST; j += 64) atomicAdd(&a.tile_count[j], 1);
    return;
  }
  // A (maxima above m*) and the first k - |A| tiles whose maximum is m*, in
  // tile index order (the selection relies on it: candidate order is then id
  // order)
  int gt = 0;
#pragma unroll
  for (int u = 0; u < CW_MPL; ++u) gt += __popcll(__ballot(key[u] > K));
  const int need = k - gt;
  int *tiles = a.cand_tile + (size_t)t * C;
  const uint64_t lt = (1ull << lane) - 1ull;
  int n = 0, taken = 0;   // tiles written; tied tiles met (both uniform)
#pragma unroll
  for (int u = 0; u < CW_MPL; ++u) {
    const bool tie = key[u] == K;
    const uint64_t bt = __ballot(tie);
    const bool f = key[u] > K || (tie && taken + __popcll(bt & lt) < need);
    const uint64_t b = __ballot(f);
    if (f) {
      const int j = 64 * u + lane;
      tiles[n + __popcll(b & lt)] = j;
      atomicAdd(&a.tile_count[j], 1);
    }
    n += __popcll(b);
    taken += __popcll(bt);
  }
  if (lane == 0) a.cand_n[t] = n;
}

// CPL >= 2 k, even: candidate i = 64 u + lane of the
// row's k x 128, entry i & 127 of tile list[i >> 7].  The list is in tile
// order, so candidate order is id order: the ties at the k-th value are cut
// at the smallest candidate indices, and ids are looked up for the winners
// only.  Entries past V hold NaN (stored so by the tile-logits kernel).
template <int CPL>
__global__ __launch_bounds__(256) void topk_select_wave_kernel(const TopkDirectArgs a) {
  __shared__ float win_v[4][64];
  __shared__ int win_i[4][64];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + w;   // uniform over the wave
  if (t >= a.T) return;
  const int cn = a.cand_n[t];
  if (cn < 0) return;   // a row that needs all its tiles: the workgroup kernel
  const int k = a.k;
  const int ne = cn * STAT_V;
  const float *zp = a.pair_z + (size_t)t * a.C * STAT_V;
  const float itau = a.inv_tau;
  const bool rb16 = a.bf16 != 0;
  uint32_t key[CPL];   // 0: no candidate (past the row's k x 128, or NaN)
#pragma unroll
  for (int u = 0; u < CPL; ++u) {
    const int i = 64 * u + lane;
    float z = zp[i < ne ? i : 0] * itau;   // an unconditional load, then the select
    if (rb16) z = (float)(__bf16)z;
    key[u] = (i < ne && z == z) ? order_key(z) : 0u;
  }
  // (every predicate below is false for key 0: the thresholds are >= 1 and
  // K >= 1 once kk > 0; no separate validity mask per candidate)
  auto count = [&](auto pred) {   // over the wave, in the scalar unit
    int c = 0;
#pragma unroll
    for (int u = 0; u < CPL; ++u) c += __popcll(__ballot(pred(u)));
    return c;
  };
  const int nvalid = count([&](int u) { return key[u] >= 1u; });
  const int kk = k < nvalid ? k : nvalid;
  uint32_t K = 0;   // the largest key with at least kk entries at or above it
  int x = 0;        // ties at K are taken for candidate indices <= x
  if (kk > 0) {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t trial = K | (1u << bit);
      if (count([&](int u) { return key[u] >= trial; }) >= kk) K = trial;
    }
    const int need = kk - count([&](int u) { return key[u] > K; });
    const int top = ne > 1 ? 31 - __clz(ne - 1) : 0;
    for (int bit = top; bit >= 0; --bit) {
      const int trial = x | (1 << bit);
      // candidate 64 u + lane < trial  <=>  lane < trial - 64 u (a scalar per u)
      if (count([&](int u) { return key[u] == K && lane < trial - 64 * u; }) < need) x = trial;
    }
  }
  // the kk winners into this wave's slots, in any order
  const uint64_t lt = (1ull << lane) - 1ull;
  const int *list = a.cand_tile + (size_t)t * a.C;
  // the winners' values are read again (a fresh load: keeping the first
  // loop's values live would cost CPL registers)
  const float *zw = zp;
  asm volatile("" : "+s"(zw));
  int nw = 0;
#pragma unroll
  for (int u = 0; u < CPL; ++u) {
    const bool f = kk > 0 && (key[u] > K || (key[u] == K && lane <= x - 64 * u));
    const uint64_t b = __ballot(f);
    if (f) {
      const int i = 64 * u + lane;
      const int at = nw + __popcll(b & lt);
      float z = zw[i] * itau;
      if (rb16) z = (float)(__bf16)z;
      win_v[w][at] = z;
      win_i[w][at] = list[i / STAT_V] * STAT_V + (i % STAT_V);
    }
    nw += __popcll(b);
  }
  __builtin_amdgcn_wave_barrier();
  const float l = a.lse[t];
  if (lane < kk) {
    const float mv = win_v[w][lane];
    const int mi = win_i[w][lane];
    int rank = 0;
    for (int q = 0; q < kk; ++q) rank += cand_gt(win_v[w][q], win_i[w][q], mv, mi) ? 1 : 0;
    a.out_lp[(size_t)t * k + rank] = mv - l;
    a.out_id[(size_t)t * k + rank] = mi;
  } else if (lane < k) {
    a.out_lp[(size_t)t * k + lane] = -INFINITY;
    a.out_id[(size_t)t * k + lane] = -1;
  }
}

// (the kernels wrap the body: a template kernel with this body itself left
// its host-side launch stubs unemitted)
template <int NW>
__global__ __launch_bounds__(64 * NW, 4) void tile_logits_kernel(const TopkDirectArgs a) {
  __shared__ __attribute__((aligned(16))) TileStage wlds[2];
  tile_logits_body<NW>(a, wlds);
}

void launch_tile_logits(const TopkDirectArgs &a, hipStream_t s) {
  if (a.tl_pairs == 256)
    hipLaunchKernelGGL((tile_logits_kernel<8>), dim3(a.items_max), dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL((tile_logits_kernel<4>), dim3(a.items_max), dim3(256), 0, s, a);
}

template <int KC>
void launch_topk_direct_kc(const TopkDirectArgs &a, hipStream_t s) {
  const int wave_blocks = ceil_div(a.T, 4);
  // up to 64 x CW_MPL tiles: a wave per row for the candidates (their lists
  // in tile order) and for the selection of the rows with k candidate tiles
  const bool waves = a.nST <= 64 * CW_MPL;
  if (waves)
    hipLaunchKernelGGL(topk_cand_wave_kernel, dim3(wave_blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((topk_cand_kernel<KC>), dim3(a.T), dim3(TOPK_THREADS), 0, s, a);
  hipLaunchKernelGGL(topk_plan_kernel, dim3(1), dim3(PLAN_THREADS), 0, s, a);
  hipLaunchKernelGGL(topk_scatter_kernel, dim3(a.T), dim3(64), 0, s, a);
  launch_tile_logits(a, s);
  // the selection: a wave per row up to k = 32 (2 k candidates per lane in
  // registers; for k = 64 the workgroup kernel measured faster)
  const bool wave_sel = waves && a.k <= 32;
  if (wave_sel) {
    if (a.k <= 8)
      hipLaunchKernelGGL(topk_select_wave_kernel<16>, dim3(wave_blocks), dim3(256), 0, s, a);
    else if (a.k <= 16)
      hipLaunchKernelGGL(topk_select_wave_kernel<32>, dim3(wave_blocks), dim3(256), 0, s, a);
    else if (a.k <= 24)
      hipLaunchKernelGGL(topk_select_wave_kernel<48>, dim3(wave_blocks), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(topk_select_wave_kernel<64>, dim3(wave_blocks), dim3(256), 0, s, a);
  }
  // the rows that need all their tiles (and, without the wave kernels, all rows)
  const PairSrc ps{a.cand_n, a.cand_tile, a.deg_rank, a.pair_z, a.C, wave_sel ? 1 : 0};
  hipLaunchKernelGGL((topk_kernel<KC, true>), dim3(a.T), dim3(TOPK_THREADS), 0, s, nullptr,
                     (int64_t)0, a.lse, a.part_m, a.T, a.V, a.nST, a.k, a.inv_tau, a.bf16,
                     a.out_lp, a.out_id, ps);
}

hipError_t launch_topk_direct(const TopkDirectArgs &a, hipStream_t s) {
  hipError_t e = launch_zero(reinterpret_cast<float *>(a.tile_count), a.nST, s);
  if (e != hipSuccess) return e;
  if (a.k <= 8) launch_topk_direct_kc<8>(a, s);
  else if (a.k <= 16) launch_topk_direct_kc<16>(a, s);
  else if (a.k <= 32) launch_topk_direct_kc<32>(a, s);
  else launch_topk_direct_kc<64>(a, s);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void zero_kernel(float *x, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    x[i] = 0.0f;
}

hipError_t launch_zero(float *x, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256),
                     0, s, x, n);
  return hipGetLastError();
}

hipError_t launch_compare(const float *a, const float *b, int64_t n, double *stats,
                          hipStream_t s) {
  hipLaunchKernelGGL(compare_kernel, dim3(1), dim3(COMPARE_THREADS), 0, s, a, b,
                     n, stats);
  return hipGetLastError();
}

}  // namespace rlk
