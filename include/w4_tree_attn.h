/* Tree-draft verify attention: the attention step of a verify pass over a
 * draft tree of M tokens.
 *
 * The pages describe tree verification in words only (the review page
 * "Speculative Decoding Meets Quantization", "The Compatibility Problem":
 * tree verification holds several candidates and verifies them in parallel;
 * the explainer page "Speculative Decoding이란?", section 8: a tree of
 * candidates A -> B, C, D that the large model checks at once, and section
 * 10.1: Medusa's tree-based attention).  Read as: draft token i attends to
 * every position of the KV prefix and to draft token j exactly when bit j of
 * masks[i] is set (for a tree: i itself and its ancestors), with
 *   out[i][h] = sum_k softmax_k(q[i][h] . key_k * scale) value_k
 * and query head h reading key/value head h / (num_heads / num_kv_heads).
 * A token that sees no key gets 0.
 *
 * Device pointers, row-major, 16-byte aligned (masks 8):
 *   q        [M][num_heads][head_dim]      bf16 bit patterns
 *   k_cache, v_cache [L][num_kv_heads][head_dim]  bf16 (the prefix; may be NULL when L == 0)
 *   k_draft, v_draft [M][num_kv_heads][head_dim]  bf16 (the draft tokens' own keys/values)
 *   masks    [M] uint64
 *   out      [M][num_heads][head_dim]      fp32
 * scale: 0 selects 1/sqrt(head_dim).  Limits: head_dim == 128, 1 <= M <= 64
 * (M == 0 does nothing), 0 <= L <= W4_TREE_MAX_L, num_heads a multiple of
 * num_kv_heads, num_heads <= 256.
 * Arithmetic: bf16 MFMA products with fp32 accumulation, fp32 softmax, the
 * probabilities rounded to bf16 for the value product; each output is within
 * 1e-2 * sum_k p_k |value_k| of the exact result.  Deterministic.  Calls
 * share a per-device workspace (allocated once, with the arrival counters of
 * the fused merge set to zero; every call leaves them at zero): calls that
 * overlap in time on one GPU race.  Enqueued on `stream`; returns without
 * waiting.
 *
 * The key sequence is cut into splits run by separate workgroups; their
 * log-sum-exp merge runs in the last workgroup of each row tile to finish
 * (W4_TREE_MERGE_LAST) or in a second launch (W4_TREE_MERGE_LAUNCH).  The
 * default (W4_TREE_MERGE_AUTO, and w4_tree_attention) merges in the last
 * workgroup only where a tile's partial results are small (at most 16 rows
 * per key/value head and 72 KiB per tile: one or two draft tokens over a
 * short prefix with 8 query heads per key/value head), in a second launch
 * otherwise.  w4_tree_attention_plan returns the split count and the merge
 * that a call of that shape uses (W4_TREE_MERGE_AUTO when there is one split
 * and nothing to merge), without a GPU.
 * Returns W4_OK, W4_ERR_INVALID (NULL, negative, misaligned, out overlapping
 * an input, bad scale), W4_ERR_UNSUPPORTED (limits) or W4_ERR_HIP; every
 * check runs before the first HIP call.
 */
#ifndef W4_TREE_ATTN_H
#define W4_TREE_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4_TREE_MAX_M 64
#define W4_TREE_MAX_L (1 << 20)

#define W4_TREE_MERGE_AUTO 0
#define W4_TREE_MERGE_LAUNCH 1
#define W4_TREE_MERGE_LAST 2

int w4_tree_attention(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache, const uint16_t* k_draft,
                      const uint16_t* v_draft, const uint64_t* masks, int M, int L, int num_heads, int num_kv_heads,
                      int head_dim, float scale, float* out, void* stream);
/* merge: W4_TREE_MERGE_AUTO, _LAUNCH or _LAST; anything else W4_ERR_INVALID. */
int w4_tree_attention_ex(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache, const uint16_t* k_draft,
                         const uint16_t* v_draft, const uint64_t* masks, int M, int L, int num_heads,
                         int num_kv_heads, int head_dim, float scale, int merge, float* out, void* stream);
/* Host only.  M >= 1; the limits above (W4_ERR_UNSUPPORTED), negative sizes
 * or a bad merge (W4_ERR_INVALID).  splits, merge_used may be NULL. */
int w4_tree_attention_plan(int M, int L, int num_heads, int num_kv_heads, int merge, int* splits, int* merge_used);

#ifdef __cplusplus
}
#endif

#endif
