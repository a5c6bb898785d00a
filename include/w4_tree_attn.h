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
 * share a per-device workspace (allocated once): calls that overlap in time
 * on one GPU race.  Enqueued on `stream`; returns without waiting.
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

int w4_tree_attention(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache, const uint16_t* k_draft,
                      const uint16_t* v_draft, const uint64_t* masks, int M, int L, int num_heads, int num_kv_heads,
                      int head_dim, float scale, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif
