// api.hip -- the C ABI declared in include/rlk.h: argument validation,
// workspace carve-up and the kernel launches.  Validation happens before any
// HIP call, so an invalid call launches nothing and writes nothing.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "internal.h"
#include "rlk.h"

namespace {

using rlk::ceil_div;

// T and V: a tile's last row index (up to 255 past the last real row) and
// every per-row index the kernels form in int stay below 2^31.
constexpr int64_t MAX_ROWS = 2147483647 - 4095;
// Elements of rlk_compare (indexed in 64 bits on the device).
constexpr int64_t MAX_COMPARE = 2147483647;
constexpr int64_t MAX_H = 65536;
constexpr int64_t MAX_LD = int64_t(1) << 21;  // 256-row tile bytes < 2^31
// workgroup tiles: a walk's tile index plus a grid of workgroups stays below 2^31
constexpr int64_t MAX_TILES = MAX_ROWS - 4096;
// Columns of a stored fp32 output: the store kernel addresses 32 rows through
// one buffer resource, whose byte offsets must stay below 2^31.
constexpr int64_t MAX_STORE_COLS = int64_t(1) << 24;
constexpr size_t WS_ALIGN = 256;

thread_local hipError_t g_last_hip_error = hipSuccess;

bool aligned(const void *p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

size_t round_up(size_t x) { return (x + WS_ALIGN - 1) / WS_ALIGN * WS_ALIGN; }

size_t stats_bytes(int64_t T, int64_t V) {
  return round_up((size_t)ceil_div(V, rlk::STAT_V) * (size_t)T * sizeof(float));
}

// Shape and support checks shared by the GEMM entry points.
int check_shapes(int64_t T, int64_t H, int64_t V, int64_t ldh, int64_t ldw) {
  if (T < 0 || H <= 0 || V <= 0 || ldh < H || ldw < H)
    return RLK_ERR_INVALID_SHAPE;
  if (H % rlk::TILE_K != 0 || H > MAX_H || T > MAX_ROWS || V > MAX_ROWS ||
      ldh > MAX_LD || ldw > MAX_LD)
    return RLK_ERR_UNSUPPORTED;
  const int64_t tiles = (int64_t)ceil_div(T, rlk::TILE_T) * ceil_div(V, rlk::TILE_V);
  if (tiles > MAX_TILES) return RLK_ERR_UNSUPPORTED;
  return RLK_OK;
}

int check_operands(const void *hidden, int64_t ldh, const void *weight,
                   int64_t ldw) {
  if (!hidden || !weight) return RLK_ERR_NULL_POINTER;
  if (!aligned(hidden, 16) || !aligned(weight, 16) || ldh % 8 != 0 ||
      ldw % 8 != 0)
    return RLK_ERR_MISALIGNED;
  return RLK_OK;
}

// Contract options of the _ex entry points.
int check_options(float inv_tau, int flags) {
  if (!(inv_tau > 0.0f) || !(inv_tau <= 3.402823466e38f)) return RLK_ERR_INVALID_VALUE;
  if (flags & ~(RLK_LOGITS_BF16 | RLK_ENTROPY)) return RLK_ERR_INVALID_VALUE;
  return RLK_OK;
}

// Workspace: part_m, part_s, xt, then part_u when the entropy is asked for,
// then the statistics GEMM's tile-claim counters.
constexpr size_t QUEUE_BYTES = 256;
size_t part_u_offset(int64_t T, int64_t V) {
  return 2 * stats_bytes(T, V) + round_up((size_t)T * sizeof(float));
}
size_t ws_bytes_for(int64_t T, int64_t V, int flags) {
  return part_u_offset(T, V) + ((flags & RLK_ENTROPY) ? stats_bytes(T, V) : 0) + QUEUE_BYTES;
}

rlk::GemmArgs gemm_args(const void *hidden, int64_t ldh, const void *weight,
                        int64_t ldw, int64_t T, int64_t H, int64_t V) {
  rlk::GemmArgs g{};
  g.hidden = static_cast<const uint16_t *>(hidden);
  g.weight = static_cast<const uint16_t *>(weight);
  g.ldh = ldh;
  g.ldw = ldw;
  g.T = (int)T;
  g.H = (int)H;
  g.V = (int)V;
  g.nMT = ceil_div(T, rlk::TILE_T);
  g.nVT = ceil_div(V, rlk::TILE_V);
  g.nST = ceil_div(V, rlk::STAT_V);
  return g;
}

// Compute units of the current device (the persistent kernel's workgroup
// count).  Falls back to 256 (MI355X) if the query fails.
int compute_units() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return 256;
  return cus;
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return RLK_OK;
  g_last_hip_error = e;
  return RLK_ERR_HIP;
}

// Backward: workspace layout, limits and launch helpers.
int64_t pad64(int64_t x) { return (x + 63) / 64 * 64; }

// dz [T][pad64(V)] (the operand of both products) and hidden^T [H][pad64(T)]
// (grad_weight's), then the GEMMs' tile-claim counters (reset before each
// launch).  Neither the weight nor dz needs a transposed copy: grad_hidden
// reads the weight and grad_weight reads dz as stored (K-major).
struct BwdLayout {
  size_t dz, ht, queue, total;  // byte offsets and size
};

// dz serves both products; h^T only the product over the tokens.
BwdLayout bwd_layout(int64_t T, int64_t H, int64_t V, bool want_w) {
  BwdLayout L{};
  size_t o = 0;
  L.dz = o;
  o += round_up((size_t)T * pad64(V) * 2);
  L.ht = o;
  if (want_w) o += round_up((size_t)H * pad64(T) * 2);
  L.queue = o;
  o += QUEUE_BYTES;
  L.total = o;
  return L;
}

// The backward's own size limits: pad64(V) and pad64(T) are the row strides
// of dz and of the transposed copies, so both must fit the stride limit.
int check_backward(int64_t T, int64_t H, int64_t V, int64_t ldh, int64_t ldw,
                   float inv_tau) {
  int st = check_shapes(T, H, V, ldh, ldw);
  if (st != RLK_OK) return st;
  if (pad64(V) > MAX_LD || pad64(T) > MAX_LD) return RLK_ERR_UNSUPPORTED;
  return check_options(inv_tau, 0);
}

rlk::GemmArgs dz_args(const void *hidden, int64_t ldh, const void *weight, int64_t ldw,
                      const int32_t *targets, const float *lse, const float *grad, int64_t T,
                      int64_t H, int64_t V, float inv_tau) {
  rlk::GemmArgs g = gemm_args(hidden, ldh, weight, ldw, T, H, V);
  g.targets = targets;
  g.lse = lse;
  g.grad = grad;
  g.inv_tau = inv_tau;
  g.ex = 3;
  g.Vp = (int)pad64(V);
  return g;
}

// out [B rows][A rows] fp32 = A . B^T over depth K: B is [Brows][K]; A is
// [Arows][K], or with a_kr > 0 K-major, [a_kr][a_cols] with a_cols >= Arows
// (default Arows) a multiple of 8 (rows a_kr .. K-1 of the depth read as
// zeros).  out_t (K-major A only): out is stored transposed, [A rows][B rows]
// (16-byte aligned, Brows a multiple of 4).
int plain_gemm(const uint16_t *A, int64_t lda, int64_t Arows, const uint16_t *B,
               int64_t ldb, int64_t Brows, int64_t K, float *out, int *queue,
               hipStream_t s, int64_t a_kr = 0, int64_t a_cols = 0, bool out_t = false) {
  rlk::GemmArgs g = gemm_args(B, ldb, A, lda, Brows, K, Arows);
  g.kmw = a_kr > 0;
  g.kr = (int)a_kr;
  g.kcols = (int)(a_cols > 0 ? a_cols : Arows);
  g.out_t = out_t ? 1 : 0;
  g.logits = out;
  g.queue = queue;
  // Prefetching a hidden-role operand that streams from HBM (grad_hidden's
  // dz) into L2 as well as the weight role measured 3.7 % faster over the
  // whole backward, bitwise identical.  grad_weight's hidden role (h^T, T H
  // bf16) stays in the memory-side cache: without its prefetch the backward
  // measured 1.1 % faster.
  g.pf_hidden = out_t ? 0 : 1;
  return hip_status(rlk::launch_gemm_logits(g, compute_units(), s));
}

}  // namespace

extern "C" {

int rlk_abi_version(void) { return RLK_ABI_VERSION; }

int rlk_vocab_tile(void) { return rlk::STAT_V; }

int rlk_last_hip_error(void) { return (int)g_last_hip_error; }

const char *rlk_status_string(int status) {
  switch (status) {
    case RLK_OK: return "ok";
    case RLK_ERR_NULL_POINTER: return "a required pointer is NULL";
    case RLK_ERR_INVALID_SHAPE:
      return "invalid shape (T < 0, H <= 0, V <= 0, n < 0 or ld < H)";
    case RLK_ERR_UNSUPPORTED:
      return "unsupported size (H must be a multiple of 64 and <= 65536; "
             "T, V <= 2^31 - 4096; ld <= 2^21)";
    case RLK_ERR_MISALIGNED:
      return "misaligned pointer or row stride (16-byte operands, ld % 8 == 0, "
             "4-byte vectors)";
    case RLK_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case RLK_ERR_HIP: return "HIP launch error (see rlk_last_hip_error)";
    case RLK_ERR_INVALID_VALUE:
      return "invalid option (inverse temperature not finite and > 0, or unknown flag bits)";
    case RLK_ERR_SCRATCH_LIMIT:
      return "T and V need more workspace than the allocation-free entry point's static "
             "scratch (RLK_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

size_t rlk_workspace_bytes_ex(int64_t T, int64_t V, int flags) {
  if (T <= 0 || V <= 0 || T > MAX_ROWS || V > MAX_ROWS) return 0;
  if (check_options(1.0f, flags) != RLK_OK) return 0;
  return ws_bytes_for(T, V, flags);
}

int rlk_workspace_layout(int64_t T, int64_t V, int flags, size_t *off_m, size_t *off_s,
                         size_t *off_xt, size_t *off_u) {
  if (T <= 0 || V <= 0) return RLK_ERR_INVALID_SHAPE;
  if (T > MAX_ROWS || V > MAX_ROWS) return RLK_ERR_UNSUPPORTED;
  if (check_options(1.0f, flags) != RLK_OK) return RLK_ERR_INVALID_VALUE;
  // the carve-up every entry point uses (rlk_vocab_stats_ex, rlk_vocab_merge_ex)
  if (off_m) *off_m = 0;
  if (off_s) *off_s = stats_bytes(T, V);
  if (off_xt) *off_xt = 2 * stats_bytes(T, V);
  if (off_u) *off_u = part_u_offset(T, V);
  return RLK_OK;
}

size_t rlk_selected_logp_workspace_bytes(int64_t T, int64_t H, int64_t V) {
  if (H <= 0) return 0;   // H does not change the size, but must be a size
  return rlk_workspace_bytes_ex(T, V, 0);
}

int rlk_vocab_stats_ex(const void *hidden, int64_t ld_hidden, const void *weight_shard,
                       int64_t ld_weight, const int32_t *targets, int64_t T, int64_t H,
                       int64_t V, int64_t v_begin, int64_t v_count, float inv_temperature,
                       int flags, void *workspace, size_t workspace_bytes, void *stream) {
  int st = check_shapes(T, H, V, ld_hidden, ld_weight);
  if (st != RLK_OK) return st;
  st = check_options(inv_temperature, flags);
  if (st != RLK_OK) return st;
  if (v_begin < 0 || v_count <= 0 || v_begin > V - v_count) return RLK_ERR_INVALID_SHAPE;
  // Slices start on a workgroup column and all but the last are whole columns,
  // so every statistics tile is computed exactly as in the unsliced call.
  if (v_begin % rlk::TILE_V != 0 || (v_begin + v_count != V && v_count % rlk::TILE_V != 0))
    return RLK_ERR_UNSUPPORTED;
  if (T == 0) return RLK_OK;
  st = check_operands(hidden, ld_hidden, weight_shard, ld_weight);
  if (st != RLK_OK) return st;
  if (!targets || !workspace) return RLK_ERR_NULL_POINTER;
  if (!aligned(targets, 4) || !aligned(workspace, 16)) return RLK_ERR_MISALIGNED;
  if (workspace_bytes < ws_bytes_for(T, V, flags)) return RLK_ERR_WORKSPACE_TOO_SMALL;
  char *ws = static_cast<char *>(workspace);
  rlk::GemmArgs g = gemm_args(hidden, ld_hidden, weight_shard, ld_weight, T, H, v_count);
  g.targets = targets;
  g.part_m = reinterpret_cast<float *>(ws);
  g.part_s = reinterpret_cast<float *>(ws + stats_bytes(T, V));
  g.xt = reinterpret_cast<float *>(ws + 2 * stats_bytes(T, V));
  g.part_u = reinterpret_cast<float *>(ws + part_u_offset(T, V));
  // Dynamic tile claims for the whole vocabulary only: slices of one
  // workspace may run at the same time on several streams.
  g.queue = (v_begin == 0 && v_count == V)
                ? reinterpret_cast<int *>(ws + ws_bytes_for(T, V, flags) - QUEUE_BYTES)
                : nullptr;
  g.js_base = (int)(v_begin / rlk::STAT_V);
  g.y_base = (int)v_begin;
  g.inv_tau = inv_temperature;
  g.bf16_logits = (flags & RLK_LOGITS_BF16) ? 1 : 0;
  // The plain kernel when no option changes a logit (its bits are those of
  // the option kernel at inv_tau = 1 without rounding; the tests check it).
  g.ex = (flags & RLK_ENTROPY) ? 2 : (inv_temperature != 1.0f || g.bf16_logits) ? 1 : 0;
  return hip_status(rlk::launch_gemm_stats(g, compute_units(), static_cast<hipStream_t>(stream)));
}

int rlk_vocab_stats_shard(const void *hidden, int64_t ld_hidden,
                          const void *weight_shard, int64_t ld_weight,
                          const int32_t *targets, int64_t T, int64_t H, int64_t V,
                          int64_t v_begin, int64_t v_count, void *workspace,
                          size_t workspace_bytes, void *stream) {
  return rlk_vocab_stats_ex(hidden, ld_hidden, weight_shard, ld_weight, targets, T, H, V,
                            v_begin, v_count, 1.0f, 0, workspace, workspace_bytes, stream);
}

int rlk_vocab_stats(const void *hidden, int64_t ld_hidden, const void *weight,
                    int64_t ld_weight, const int32_t *targets, int64_t T,
                    int64_t H, int64_t V, void *workspace,
                    size_t workspace_bytes, void *stream) {
  return rlk_vocab_stats_shard(hidden, ld_hidden, weight, ld_weight, targets, T, H, V, 0, V,
                               workspace, workspace_bytes, stream);
}

int rlk_vocab_merge_ex(const int32_t *targets, float *logp, float *lse, float *entropy,
                       int64_t T, int64_t V, int flags, const void *workspace,
                       size_t workspace_bytes, void *stream) {
  if (T < 0 || V <= 0) return RLK_ERR_INVALID_SHAPE;
  if (T > MAX_ROWS || V > MAX_ROWS) return RLK_ERR_UNSUPPORTED;
  if (check_options(1.0f, flags) != RLK_OK) return RLK_ERR_INVALID_VALUE;
  if (T == 0) return RLK_OK;
  const bool ent = (flags & RLK_ENTROPY) != 0;
  if (!targets || !logp || !lse || !workspace || (ent && !entropy)) return RLK_ERR_NULL_POINTER;
  if (!aligned(targets, 4) || !aligned(logp, 4) || !aligned(lse, 4) ||
      !aligned(workspace, 16) || (ent && !aligned(entropy, 4)))
    return RLK_ERR_MISALIGNED;
  if (workspace_bytes < ws_bytes_for(T, V, flags)) return RLK_ERR_WORKSPACE_TOO_SMALL;
  const char *ws = static_cast<const char *>(workspace);
  rlk::MergeArgs mg{};
  mg.part_m = reinterpret_cast<const float *>(ws);
  mg.part_s = reinterpret_cast<const float *>(ws + stats_bytes(T, V));
  mg.xt = reinterpret_cast<const float *>(ws + 2 * stats_bytes(T, V));
  mg.part_u = ent ? reinterpret_cast<const float *>(ws + part_u_offset(T, V)) : nullptr;
  mg.entropy = ent ? entropy : nullptr;
  mg.targets = targets;
  mg.logp = logp;
  mg.lse = lse;
  mg.T = (int)T;
  mg.V = (int)V;
  mg.nST = ceil_div(V, rlk::STAT_V);
  return hip_status(rlk::launch_merge(mg, static_cast<hipStream_t>(stream)));
}

int rlk_vocab_merge(const int32_t *targets, float *logp, float *lse, int64_t T,
                    int64_t V, const void *workspace, size_t workspace_bytes,
                    void *stream) {
  return rlk_vocab_merge_ex(targets, logp, lse, nullptr, T, V, 0, workspace,
                            workspace_bytes, stream);
}

int rlk_selected_logp_ex(const void *hidden, int64_t ld_hidden, const void *weight,
                         int64_t ld_weight, const int32_t *targets, float *logp,
                         float *lse, float *entropy, int64_t T, int64_t H, int64_t V,
                         float inv_temperature, int flags, void *workspace,
                         size_t workspace_bytes, void *stream) {
  // Validate everything both stages need before launching the first one.
  int st = check_shapes(T, H, V, ld_hidden, ld_weight);
  if (st != RLK_OK) return st;
  st = check_options(inv_temperature, flags);
  if (st != RLK_OK) return st;
  if (T == 0) return RLK_OK;
  st = check_operands(hidden, ld_hidden, weight, ld_weight);
  if (st != RLK_OK) return st;
  const bool ent = (flags & RLK_ENTROPY) != 0;
  if (!targets || !logp || !lse || !workspace || (ent && !entropy)) return RLK_ERR_NULL_POINTER;
  if (!aligned(logp, 4) || !aligned(lse, 4) || (ent && !aligned(entropy, 4)))
    return RLK_ERR_MISALIGNED;
  st = rlk_vocab_stats_ex(hidden, ld_hidden, weight, ld_weight, targets, T, H, V, 0, V,
                          inv_temperature, flags, workspace, workspace_bytes, stream);
  if (st != RLK_OK) return st;
  return rlk_vocab_merge_ex(targets, logp, lse, entropy, T, V, flags, workspace,
                            workspace_bytes, stream);
}

int rlk_selected_logp(const void *hidden, int64_t ld_hidden,
                      const void *weight, int64_t ld_weight,
                      const int32_t *targets, float *logp, float *lse,
                      int64_t T, int64_t H, int64_t V, void *workspace,
                      size_t workspace_bytes, void *stream) {
  return rlk_selected_logp_ex(hidden, ld_hidden, weight, ld_weight, targets, logp, lse,
                              nullptr, T, H, V, 1.0f, 0, workspace, workspace_bytes, stream);
}


// ---------------------------------------------------------------- backward --

size_t rlk_selected_logp_backward_workspace_bytes(int64_t T, int64_t H, int64_t V) {
  if (T <= 0 || H <= 0 || V <= 0 || T > MAX_ROWS || V > MAX_ROWS || H > MAX_H) return 0;
  return bwd_layout(T, H, V, true).total;
}

int rlk_logp_grad_logits(const void *hidden, int64_t ld_hidden, const void *weight,
                         int64_t ld_weight, const int32_t *targets, const float *lse,
                         const float *grad_logp, void *dz, int64_t ld_dz, int64_t T,
                         int64_t H, int64_t V, float inv_temperature, void *stream) {
  int st = check_backward(T, H, V, ld_hidden, ld_weight, inv_temperature);
  if (st != RLK_OK) return st;
  if (ld_dz < pad64(V)) return RLK_ERR_INVALID_SHAPE;
  if (ld_dz > MAX_LD) return RLK_ERR_UNSUPPORTED;
  if (T == 0) return RLK_OK;
  st = check_operands(hidden, ld_hidden, weight, ld_weight);
  if (st != RLK_OK) return st;
  if (!targets || !lse || !grad_logp || !dz) return RLK_ERR_NULL_POINTER;
  if (!aligned(targets, 4) || !aligned(lse, 4) || !aligned(grad_logp, 4) || !aligned(dz, 16) ||
      ld_dz % 8 != 0)
    return RLK_ERR_MISALIGNED;
  rlk::GemmArgs g = dz_args(hidden, ld_hidden, weight, ld_weight, targets, lse, grad_logp, T,
                            H, V, inv_temperature);
  g.dz = static_cast<uint16_t *>(dz);
  g.ld_dz = ld_dz;
  return hip_status(rlk::launch_gemm_stats(g, compute_units(), static_cast<hipStream_t>(stream)));
}

int rlk_selected_logp_backward(const void *hidden, int64_t ld_hidden, const void *weight,
                               int64_t ld_weight, const int32_t *targets, const float *lse,
                               const float *grad_logp, float *grad_hidden, float *grad_weight,
                               int64_t T, int64_t H, int64_t V, float inv_temperature,
                               void *workspace, size_t workspace_bytes, void *stream) {
  int st = check_backward(T, H, V, ld_hidden, ld_weight, inv_temperature);
  if (st != RLK_OK) return st;
  const bool want_h = grad_hidden != nullptr, want_w = grad_weight != nullptr;
  if (!want_h && !want_w) return RLK_OK;
  if ((want_h && !aligned(grad_hidden, 4)) || (want_w && !aligned(grad_weight, 16)))
    return RLK_ERR_MISALIGNED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 0) {  // no rows: grad_weight is a sum over nothing
    return want_w ? hip_status(rlk::launch_zero(grad_weight, V * H, s)) : RLK_OK;
  }
  st = check_operands(hidden, ld_hidden, weight, ld_weight);
  if (st != RLK_OK) return st;
  if (!targets || !lse || !grad_logp || !workspace) return RLK_ERR_NULL_POINTER;
  if (!aligned(targets, 4) || !aligned(lse, 4) || !aligned(grad_logp, 4) ||
      !aligned(workspace, 16))
    return RLK_ERR_MISALIGNED;
  const BwdLayout L = bwd_layout(T, H, V, want_w);
  if (workspace_bytes < L.total) return RLK_ERR_WORKSPACE_TOO_SMALL;
  char *ws = static_cast<char *>(workspace);
  const int64_t Vp = pad64(V), Tp = pad64(T);
  uint16_t *dz = reinterpret_cast<uint16_t *>(ws + L.dz);
  uint16_t *ht = reinterpret_cast<uint16_t *>(ws + L.ht);
  const uint16_t *h16 = static_cast<const uint16_t *>(hidden);
  const uint16_t *w16 = static_cast<const uint16_t *>(weight);
  // grad_weight contracts over T.  It is formed as its transpose, [H][V] =
  // h^T [H][Tp] . dz [Tp][Vp], stored transposed: dz is read K-major as the
  // dz pass wrote it (token rows are the depth), and hidden^T is a copy
  // with the tokens contiguous (T H bf16, small next to dz), so only one
  // operand takes the transposing LDS reads and no dz^T is written.  (Both
  // operands read K-major measured 0.56 ms slower than a dz^T store plus
  // this copy; a dz^T store measured slower than this product.)
  if (want_w) {
    st = hip_status(rlk::launch_transpose(h16, ld_hidden, (int)T, (int)H, ht, Tp, s));
    if (st != RLK_OK) return st;
  }
  rlk::GemmArgs g = dz_args(hidden, ld_hidden, weight, ld_weight, targets, lse, grad_logp, T,
                            H, V, inv_temperature);
  g.dz = dz;
  g.ld_dz = Vp;
  int *queue = reinterpret_cast<int *>(ws + L.queue);
  g.queue = queue;
  st = hip_status(rlk::launch_gemm_stats(g, compute_units(), s));
  if (st != RLK_OK) return st;
  // grad_hidden [T][H] = dz [T][Vp] . W [V][H], the weight read K-major as
  // stored (its rows are the depth; rows V .. Vp-1 read as zeros): no
  // transposed copy of the weight (a 2 x V x H byte round trip)
  if (want_h) {
    st = plain_gemm(w16, ld_weight, H, dz, Vp, T, Vp, grad_hidden, queue, s, V);
    if (st != RLK_OK) return st;
  }
  // grad_weight [V][H] = (ht [H][Tp] . dz [Tp][Vp])^T: dz in the weight role,
  // K-major with T depth rows (rows T .. Tp-1 read as zeros) and Vp columns
  // (columns V .. Vp-1 hold zeros), the output stored transposed
  if (want_w) st = plain_gemm(dz, Vp, V, ht, Tp, H, Tp, grad_weight, queue, s, T, Vp, true);
  return st;
}

int rlk_rmsnorm(const void *x, int64_t ld_x, const void *gamma, float eps, void *y,
                int64_t ld_y, int64_t T, int64_t H, void *stream) {
  if (T < 0 || H <= 0 || ld_x < H || ld_y < H) return RLK_ERR_INVALID_SHAPE;
  if (H % 8 != 0 || T > MAX_ROWS || ld_x > MAX_LD || ld_y > MAX_LD) return RLK_ERR_UNSUPPORTED;
  if (!(eps >= 0.0f) || !(eps <= 3.402823466e38f)) return RLK_ERR_INVALID_VALUE;
  if (T == 0) return RLK_OK;
  if (!x || !gamma || !y) return RLK_ERR_NULL_POINTER;
  if (!aligned(x, 16) || !aligned(gamma, 16) || !aligned(y, 16) || ld_x % 8 != 0 ||
      ld_y % 8 != 0)
    return RLK_ERR_MISALIGNED;
  return hip_status(rlk::launch_rmsnorm(static_cast<const uint16_t *>(x), ld_x,
                                        static_cast<const uint16_t *>(gamma), eps,
                                        static_cast<uint16_t *>(y), ld_y, (int)T, (int)H,
                                        static_cast<hipStream_t>(stream)));
}

int rlk_topk_logp(const float *logits, int64_t ld_logits, const float *lse,
                  const void *workspace, size_t workspace_bytes, int64_t T, int64_t V, int k,
                  float inv_temperature, int flags, float *topk_logp, int32_t *topk_ids,
                  void *stream) {
  if (T < 0 || V <= 0 || ld_logits < V) return RLK_ERR_INVALID_SHAPE;
  if (T > MAX_ROWS || V > MAX_ROWS) return RLK_ERR_UNSUPPORTED;
  if (check_options(inv_temperature, flags) != RLK_OK || k < 1 || k > 64 || k > V)
    return RLK_ERR_INVALID_VALUE;
  if (T == 0) return RLK_OK;
  if (!logits || !lse || !workspace || !topk_logp || !topk_ids) return RLK_ERR_NULL_POINTER;
  if (!aligned(logits, 4) || !aligned(lse, 4) || !aligned(workspace, 16) ||
      !aligned(topk_logp, 4) || !aligned(topk_ids, 4))
    return RLK_ERR_MISALIGNED;
  if (workspace_bytes < stats_bytes(T, V)) return RLK_ERR_WORKSPACE_TOO_SMALL;
  return hip_status(rlk::launch_topk(logits, ld_logits, lse,
                                     static_cast<const float *>(workspace), (int)T, (int)V, k,
                                     inv_temperature, (flags & RLK_LOGITS_BF16) ? 1 : 0,
                                     topk_logp, topk_ids, static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------ top-k from the operands
}  // extern "C"

namespace {

struct TopkLayout {
  size_t pair_z, bucket, cand_tile, cand_n, deg_rank, deg_row, tile_count, tile_off, tile_fill,
      item_off, item_tile, totals, total;
  int64_t P, items_max;
};

// The direct top-k's workspace: k pair slots per row (128 fp32 logits each),
// then room for dcap rows with m* = -inf (all nST tiles each) when nST > k;
// the pair buckets, the per-row candidate lists, and the plan's tile tables.
TopkLayout topk_layout(int64_t T, int64_t V, int64_t k, int64_t dcap) {
  TopkLayout L{};
  const int64_t nST = ceil_div(V, rlk::STAT_V);
  if (nST <= k) dcap = 0;   // such rows use their own k slots
  L.P = T * k + dcap * nST;
  // work items of up to 128 pairs of a tile (256 when k > 32: about twice
  // the pairs per tile, the weights then streamed once per tile)
  const int64_t per_item = k > 32 ? 256 : 128;
  L.items_max = (L.P + per_item - 1) / per_item + nST;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += round_up(bytes);
    return at;
  };
  L.pair_z = take((size_t)L.P * rlk::STAT_V * 4);
  L.bucket = take((size_t)L.P * 4);
  L.cand_tile = take((size_t)T * k * 4);
  L.cand_n = take((size_t)T * 4);
  L.deg_rank = take((size_t)T * 4);
  L.deg_row = take((size_t)(dcap > 0 ? dcap : 1) * 4);
  L.tile_count = take((size_t)nST * 4);
  L.tile_off = take((size_t)nST * 4);
  L.tile_fill = take((size_t)nST * 4);
  L.item_off = take((size_t)(nST + 1) * 4);
  L.item_tile = take((size_t)L.items_max * 4);
  L.totals = take(16);
  L.total = o;
  return L;
}

// Pair and item indices are int on the device.
constexpr int64_t MAX_PAIRS = int64_t(1) << 30;

int check_topk_direct(int64_t T, int64_t V, int k, int64_t dcap) {
  if (dcap < 0) return RLK_ERR_INVALID_VALUE;
  if (k < 1 || k > 64 || k > V) return RLK_ERR_INVALID_VALUE;
  const int64_t nST = ceil_div(V, rlk::STAT_V);
  if (T * k + (nST > k ? dcap * nST : 0) > MAX_PAIRS) return RLK_ERR_UNSUPPORTED;
  return RLK_OK;
}

}  // namespace

extern "C" {

size_t rlk_topk_logp_direct_workspace_bytes(int64_t T, int64_t V, int k,
                                            int64_t max_degenerate_rows) {
  if (T <= 0 || V <= 0 || T > MAX_ROWS || V > MAX_ROWS) return 0;
  if (check_topk_direct(T, V, k, max_degenerate_rows) != RLK_OK) return 0;
  return topk_layout(T, V, k, max_degenerate_rows).total;
}

int rlk_topk_logp_direct(const void *hidden, int64_t ld_hidden, const void *weight,
                         int64_t ld_weight, const float *lse, const void *stats_workspace,
                         size_t stats_workspace_bytes, int64_t T, int64_t H, int64_t V, int k,
                         float inv_temperature, int flags, int64_t max_degenerate_rows,
                         void *workspace, size_t workspace_bytes, float *topk_logp,
                         int32_t *topk_ids, void *stream) {
  int st = check_shapes(T, H, V, ld_hidden, ld_weight);
  if (st != RLK_OK) return st;
  if (check_options(inv_temperature, flags) != RLK_OK) return RLK_ERR_INVALID_VALUE;
  st = check_topk_direct(T, V, k, max_degenerate_rows);
  if (st != RLK_OK) return st;
  if (T == 0) return RLK_OK;
  st = check_operands(hidden, ld_hidden, weight, ld_weight);
  if (st != RLK_OK) return st;
  if (!lse || !stats_workspace || !workspace || !topk_logp || !topk_ids)
    return RLK_ERR_NULL_POINTER;
  if (!aligned(lse, 4) || !aligned(stats_workspace, 16) || !aligned(workspace, 16) ||
      !aligned(topk_logp, 4) || !aligned(topk_ids, 4))
    return RLK_ERR_MISALIGNED;
  if (stats_workspace_bytes < stats_bytes(T, V)) return RLK_ERR_WORKSPACE_TOO_SMALL;
  const TopkLayout L = topk_layout(T, V, k, max_degenerate_rows);
  if (workspace_bytes < L.total) return RLK_ERR_WORKSPACE_TOO_SMALL;
  char *ws = static_cast<char *>(workspace);
  rlk::TopkDirectArgs a{};
  a.hidden = static_cast<const uint16_t *>(hidden);
  a.weight = static_cast<const uint16_t *>(weight);
  a.ldh = ld_hidden;
  a.ldw = ld_weight;
  a.lse = lse;
  a.part_m = static_cast<const float *>(stats_workspace);
  a.out_lp = topk_logp;
  a.out_id = topk_ids;
  a.pair_z = reinterpret_cast<float *>(ws + L.pair_z);
  a.bucket = reinterpret_cast<int *>(ws + L.bucket);
  a.cand_tile = reinterpret_cast<int *>(ws + L.cand_tile);
  a.cand_n = reinterpret_cast<int *>(ws + L.cand_n);
  a.deg_rank = reinterpret_cast<int *>(ws + L.deg_rank);
  a.deg_row = reinterpret_cast<int *>(ws + L.deg_row);
  a.tile_count = reinterpret_cast<int *>(ws + L.tile_count);
  a.tile_off = reinterpret_cast<int *>(ws + L.tile_off);
  a.tile_fill = reinterpret_cast<int *>(ws + L.tile_fill);
  a.item_off = reinterpret_cast<int *>(ws + L.item_off);
  a.item_tile = reinterpret_cast<int *>(ws + L.item_tile);
  a.totals = reinterpret_cast<int *>(ws + L.totals);
  a.inv_tau = inv_temperature;
  a.bf16 = (flags & RLK_LOGITS_BF16) ? 1 : 0;
  a.T = (int)T;
  a.H = (int)H;
  a.V = (int)V;
  a.nST = ceil_div(V, rlk::STAT_V);
  a.k = k;
  a.C = k;
  a.dcap = (int)max_degenerate_rows;
  a.tl_pairs = k > 32 ? 256 : 128;
  a.items_max = (int)L.items_max;
  return hip_status(rlk::launch_topk_direct(a, static_cast<hipStream_t>(stream)));
}

int rlk_debug_logits(const void *hidden, int64_t ld_hidden, const void *weight,
                     int64_t ld_weight, float *logits, int64_t T, int64_t H, int64_t V,
                     void *stream) {
  int st = check_shapes(T, H, V, ld_hidden, ld_weight);
  if (st != RLK_OK) return st;
  if (V > MAX_STORE_COLS) return RLK_ERR_UNSUPPORTED;
  if (T == 0) return RLK_OK;
  st = check_operands(hidden, ld_hidden, weight, ld_weight);
  if (st != RLK_OK) return st;
  if (!logits) return RLK_ERR_NULL_POINTER;
  if (!aligned(logits, 4)) return RLK_ERR_MISALIGNED;
  rlk::GemmArgs g = gemm_args(hidden, ld_hidden, weight, ld_weight, T, H, V);
  g.logits = logits;
  return hip_status(rlk::launch_gemm_logits(g, compute_units(), static_cast<hipStream_t>(stream)));
}

int rlk_logits(const void *hidden, int64_t ld_hidden, const void *weight,
               int64_t ld_weight, float *logits, int64_t T, int64_t H,
               int64_t V, void *stream) {
  return rlk_debug_logits(hidden, ld_hidden, weight, ld_weight, logits, T, H, V, stream);
}

int rlk_compare(const float *a, const float *b, int64_t n, double *stats,
                void *stream) {
  if (n < 0) return RLK_ERR_INVALID_SHAPE;
  if (n > MAX_COMPARE) return RLK_ERR_UNSUPPORTED;
  if (!stats || (n > 0 && (!a || !b))) return RLK_ERR_NULL_POINTER;
  if (!aligned(stats, 8) || !aligned(a, 4) || !aligned(b, 4))
    return RLK_ERR_MISALIGNED;
  return hip_status(rlk::launch_compare(a, b, n, stats,
                                        static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------ allocation-free variant --
//
// rlk_selected_logp_noalloc: rlk_selected_logp with its workspace in a
// file-scope device array instead of a caller's buffer.  Each GPU the
// library runs on holds its own copy of the array (RLK_NOALLOC_SCRATCH_BYTES)
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not a device address: the device address is looked up once per device,
// with that device current, and only that address is handed to kernels.

}  // extern "C"

namespace {

__device__ __attribute__((aligned(256))) unsigned char scratch[RLK_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[MAX_DEVICES];   // device address of `scratch` per device

// The device address of the current device's copy of `scratch`.
int scratch_of_current_device(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= MAX_DEVICES) return RLK_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (!p) return RLK_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return RLK_OK;
}

}  // namespace

extern "C" {

int rlk_selected_logp_noalloc(const void *hidden, int64_t ld_hidden, const void *weight,
                              int64_t ld_weight, const int32_t *targets, float *logp,
                              float *lse, int64_t T, int64_t H, int64_t V, void *stream) {
  // every check of rlk_selected_logp, before any HIP call
  int st = check_shapes(T, H, V, ld_hidden, ld_weight);
  if (st != RLK_OK) return st;
  if (T == 0) return RLK_OK;
  if (ws_bytes_for(T, V, 0) > RLK_NOALLOC_SCRATCH_BYTES) return RLK_ERR_SCRATCH_LIMIT;
  st = check_operands(hidden, ld_hidden, weight, ld_weight);
  if (st != RLK_OK) return st;
  if (!targets || !logp || !lse) return RLK_ERR_NULL_POINTER;
  if (!aligned(targets, 4) || !aligned(logp, 4) || !aligned(lse, 4)) return RLK_ERR_MISALIGNED;
  void *ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != RLK_OK) return st;
  // the same kernels as rlk_selected_logp; the tile-claim counters in the
  // scratch are reset by a kernel at the start of every call
  return rlk_selected_logp(hidden, ld_hidden, weight, ld_weight, targets, logp, lse, T, H, V,
                           ws, RLK_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
