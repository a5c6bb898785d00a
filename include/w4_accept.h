/* Acceptance step of speculative decoding, run on the verify pass's logits.
 *
 * Defined on the explainer page "Speculative Decoding이란?"
 * (dojself04.mycafe24.com), section 3 (Leviathan et al., ICML 2023), Steps 3
 * and 4, with sections 5 (greedy output and sampled distribution equal the
 * target's) and 6 (accept in order; at the first rejection draw from a
 * corrected distribution).  Verifying K drafted tokens gives K+1 rows of
 * target logits: row j is the target's next-token distribution after the
 * prefix and the first j drafted tokens.  p and q are the softmax of target
 * and draft logits.  Drafted token j is tested against row j in order:
 *   greedy:  accepted when it is the first index of the row's maximum;
 *   sampled: accepted when u[j] < min(1, p_j(d) / q_j(d)).
 * At the first rejection (row j) the next token is row j's argmax (greedy) or
 * a draw from the residual max(0, p_j - q_j) (sampled: the residual of the
 * Leviathan et al. paper the page names -- the pages do not print the
 * corrected distribution); when all K are accepted it is row K's argmax, or a
 * draw from p_K.  A draw from weights r with uniform v is the smallest t with
 * r_0 + ... + r_t > v * sum(r) (inverse CDF); the sampled step uses v = u[K].
 *
 * All pointers are device pointers; the calls enqueue work on `stream` (a
 * hipStream_t, NULL for the default stream) and return without waiting.
 *   logits        [K+1][V] fp32, row-major, 16-byte aligned, finite
 *   draft_logits  [K][V]   fp32, row-major, 16-byte aligned, finite (sampled)
 *   draft         [K]      int32 drafted tokens; one outside [0, V) is rejected
 *   u             [K+1]    fp32 uniforms in [0, 1) (sampled)
 *   out           [2]      int32: out[0] = drafted tokens accepted (0..K),
 *                          out[1] = the next token
 * Limits: 0 <= K <= W4_ACCEPT_MAX_K, 4 <= V <= W4_ACCEPT_MAX_V, V % 4 == 0.
 * Returns W4_OK, W4_ERR_INVALID (NULL, negative, misaligned, out overlapping
 * an input), W4_ERR_UNSUPPORTED (limits) or W4_ERR_HIP; every check runs
 * before the first HIP call.  Results are deterministic (fixed reduction
 * order); the arithmetic is fp32.  Calls share one small per-device
 * workspace (allocated once): calls that overlap in time on one GPU race.
 */
#ifndef W4_ACCEPT_H
#define W4_ACCEPT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4_ACCEPT_MAX_K 64
#define W4_ACCEPT_MAX_V (1 << 24)

int w4_accept_greedy(const float* logits, const int32_t* draft, int K, int V, int32_t* out, void* stream);

int w4_accept_sample(const float* logits, const float* draft_logits, const int32_t* draft, const float* u, int K,
                     int V, int32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif
