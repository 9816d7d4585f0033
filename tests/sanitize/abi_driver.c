/* Drives every validation path of the C ABI (include/rlk.h) that returns
 * before the first HIP call -- null pointers, bad shapes, sizes above the
 * limits, misalignment, short workspaces -- plus the size and layout
 * queries, in a build whose host code carries -fsanitize=address,undefined.
 * No kernel is launched: every call here is refused by validation (or has
 * no rows), so the driver runs without a GPU.  Exit status 0 when every
 * status is the documented one. */
#include <stdint.h>
#include <stdio.h>

#include "rlk.h"

static int failures = 0;
#define EXPECT(call, want)                                                      \
    do {                                                                        \
        int got_ = (call);                                                      \
        if (got_ != (want)) {                                                   \
            fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, \
                    #call, got_, (want));                                       \
            ++failures;                                                         \
        }                                                                       \
    } while (0)

int main(void) {
    void *F = (void *)(uintptr_t)0x10000;    /* aligned, never dereferenced */
    void *F2 = (void *)(uintptr_t)0x10002;   /* 2-byte aligned */
    const int32_t *Y = (const int32_t *)F;
    float *O = (float *)F;
    const size_t big = (size_t)1 << 40;
    const int64_t H = 256, V = 1000, T = 4;

    EXPECT(rlk_abi_version(), RLK_ABI_VERSION);
    for (int s = -1; s < 12; ++s)
        if (!rlk_status_string(s)) ++failures;
    EXPECT(rlk_selected_logp_workspace_bytes(0, H, V) == 0, 1);
    EXPECT(rlk_selected_logp_workspace_bytes(T, 0, V) == 0, 1);
    EXPECT(rlk_selected_logp_workspace_bytes(T, H, V) > 0, 1);
    EXPECT(rlk_selected_logp_workspace_bytes((int64_t)1 << 31, H, V) == 0, 1);
    size_t m, s, x, u;
    EXPECT(rlk_workspace_layout(T, V, 0, &m, &s, &x, &u), RLK_OK);
    EXPECT(m == 0 && s > 0 && x > s && u > x, 1);
    EXPECT(rlk_workspace_layout(T, V, 0, NULL, NULL, NULL, NULL), RLK_OK);
    EXPECT(rlk_workspace_layout(0, V, 0, &m, &s, &x, &u), RLK_ERR_INVALID_SHAPE);
    EXPECT(rlk_workspace_layout(T, V, 99, &m, &s, &x, &u), RLK_ERR_INVALID_VALUE);
    EXPECT(rlk_workspace_bytes_ex(T, V, RLK_ENTROPY) > rlk_workspace_bytes_ex(T, V, 0), 1);

    /* the hot path */
    EXPECT(rlk_selected_logp(F, H, F, H, Y, O, O, -1, H, V, F, big, NULL), RLK_ERR_INVALID_SHAPE);
    EXPECT(rlk_selected_logp(F, 100, F, H, Y, O, O, T, H, V, F, big, NULL), RLK_ERR_INVALID_SHAPE);
    EXPECT(rlk_selected_logp(F, 256, F, 256, Y, O, O, T, 192 + 8, V, F, big, NULL),
           RLK_ERR_UNSUPPORTED);
    EXPECT(rlk_selected_logp(F, H, F, H, Y, O, O, ((int64_t)1 << 31) - 4095, H, 64, F, big, NULL),
           RLK_ERR_UNSUPPORTED);
    EXPECT(rlk_selected_logp(NULL, H, F, H, Y, O, O, T, H, V, F, big, NULL), RLK_ERR_NULL_POINTER);
    EXPECT(rlk_selected_logp(F, H, F, H, NULL, O, O, T, H, V, F, big, NULL), RLK_ERR_NULL_POINTER);
    EXPECT(rlk_selected_logp(F, H, F, H, Y, O, O, T, H, V, NULL, big, NULL), RLK_ERR_NULL_POINTER);
    EXPECT(rlk_selected_logp(F2, H, F, H, Y, O, O, T, H, V, F, big, NULL), RLK_ERR_MISALIGNED);
    EXPECT(rlk_selected_logp(F, H, F, H, Y, (float *)F2, O, T, H, V, F, big, NULL),
           RLK_ERR_MISALIGNED);
    EXPECT(rlk_selected_logp(F, H, F, H, Y, O, O, T, H, V, F, 100, NULL),
           RLK_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(rlk_selected_logp(NULL, H, NULL, H, NULL, NULL, NULL, 0, H, V, NULL, 0, NULL), RLK_OK);
    EXPECT(rlk_selected_logp_noalloc(F, H, F, H, Y, O, O, 8000, H, 151936, NULL),
           RLK_ERR_SCRATCH_LIMIT);
    EXPECT(rlk_selected_logp_noalloc(F, H, F, H, NULL, O, O, T, H, V, NULL), RLK_ERR_NULL_POINTER);
    EXPECT(rlk_selected_logp_noalloc(F, 100, F, H, Y, O, O, T, H, V, NULL), RLK_ERR_INVALID_SHAPE);

    /* the stages, slices and options */
    EXPECT(rlk_vocab_stats(F, H, F, H, NULL, T, H, V, F, big, NULL), RLK_ERR_NULL_POINTER);
    EXPECT(rlk_vocab_stats(F, H, F, H, Y, T, H, V, F, 10, NULL), RLK_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(rlk_vocab_merge(Y, O, O, -3, V, F, big, NULL), RLK_ERR_INVALID_SHAPE);
    EXPECT(rlk_vocab_merge(Y, O, O, T, V, F2, big, NULL), RLK_ERR_MISALIGNED);
    EXPECT(rlk_vocab_stats_shard(F, H, F, H, Y, T, H, V, 100, 256, F, big, NULL),
           RLK_ERR_UNSUPPORTED);
    EXPECT(rlk_vocab_stats_shard(F, H, F, H, Y, T, H, V, 768, 256, F, big, NULL),
           RLK_ERR_INVALID_SHAPE);
    EXPECT(rlk_selected_logp_ex(F, H, F, H, Y, O, O, O, T, H, V, 0.0f, 0, F, big, NULL),
           RLK_ERR_INVALID_VALUE);
    EXPECT(rlk_selected_logp_ex(F, H, F, H, Y, O, O, NULL, T, H, V, 1.0f, RLK_ENTROPY, F, big,
                                NULL), RLK_ERR_NULL_POINTER);
    EXPECT(rlk_vocab_stats_ex(F, H, F, H, Y, T, H, V, 0, V, 1.0f, 8, F, big, NULL),
           RLK_ERR_INVALID_VALUE);
    EXPECT(rlk_vocab_merge_ex(Y, O, O, NULL, T, V, RLK_ENTROPY, F, big, NULL),
           RLK_ERR_NULL_POINTER);

    /* logits stage, compare, backward, rmsnorm, top-k */
    EXPECT(rlk_debug_logits(F, H, F, H, NULL, T, H, V, NULL), RLK_ERR_NULL_POINTER);
    EXPECT(rlk_debug_logits(F, H, F, H, O, T, H, ((int64_t)1 << 24) + 1, NULL),
           RLK_ERR_UNSUPPORTED);
    EXPECT(rlk_logits(F, H, F, H, (float *)F2, T, H, V, NULL), RLK_ERR_MISALIGNED);
    EXPECT(rlk_compare(O, O, -1, (double *)F, NULL), RLK_ERR_INVALID_SHAPE);
    EXPECT(rlk_compare(O, O, (int64_t)1 << 31, (double *)F, NULL), RLK_ERR_UNSUPPORTED);
    EXPECT(rlk_compare(O, O, 10, NULL, NULL), RLK_ERR_NULL_POINTER);
    EXPECT(rlk_selected_logp_backward_workspace_bytes(T, H, V) > 0, 1);
    EXPECT(rlk_selected_logp_backward(F, H, F, H, Y, O, O, O, O, T, H, V, -1.0f, F, big, NULL),
           RLK_ERR_INVALID_VALUE);
    EXPECT(rlk_selected_logp_backward(F, H, F, H, Y, O, O, O, O, T, H, V, 1.0f, F, 10, NULL),
           RLK_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(rlk_selected_logp_backward(F, H, F, H, Y, O, O, NULL, NULL, T, H, V, 1.0f, F, 10,
                                      NULL), RLK_OK);
    EXPECT(rlk_logp_grad_logits(F, H, F, H, Y, O, O, F, 64, T, H, V, 1.0f, NULL),
           RLK_ERR_INVALID_SHAPE);
    EXPECT(rlk_rmsnorm(F, H, F, 1e-6f, F, H, T, 12, NULL), RLK_ERR_UNSUPPORTED);
    EXPECT(rlk_rmsnorm(F, H, F, -1.0f, F, H, T, H, NULL), RLK_ERR_INVALID_VALUE);
    EXPECT(rlk_topk_logp(O, V, O, F, big, T, V, 65, 1.0f, 0, O, (int32_t *)F, NULL),
           RLK_ERR_INVALID_VALUE);
    EXPECT(rlk_topk_logp(O, V, O, F, 16, T, V, 5, 1.0f, 0, O, (int32_t *)F, NULL),
           RLK_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(rlk_last_hip_error(), 0);
    if (failures) {
        fprintf(stderr, "%d statuses differ\n", failures);
        return 1;
    }
    printf("abi driver: all statuses as documented\n");
    return 0;
}
