// Internal interface of the steps around the verify linear: the acceptance
// step (w4_accept.hip) and tree-draft verify attention (w4_tree_attn.hip).
// Not installed; the public ABI is include/w4_accept.h and
// include/w4_tree_attn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w4 {

// Acceptance step (w4_accept.hip).
constexpr int kAcceptMaxK = 64;                     // drafted tokens per call
constexpr int kAcceptMaxV = 1 << 24;                // vocabulary entries
constexpr size_t kAcceptWorkspaceBytes = size_t(1) << 20;
size_t accept_workspace_bytes(int K, int V);
// lt: [K+1][V] target logits, ld: [K][V] draft logits (sampled only), draft:
// [K] tokens, u: [K+1] uniforms (sampled only), out: [2] accepted count and
// next token; ws: kAcceptWorkspaceBytes.
hipError_t launch_accept(const float* lt, const float* ld, const int32_t* draft, const float* u, int K, int V,
                         int sampled, int32_t* out, void* ws, hipStream_t stream);

// Tree-draft verify attention (w4_tree_attn.hip).
constexpr int kTreeHeadDim = 128;
constexpr int kTreeMaxM = 64;
constexpr size_t kTreeWorkspaceBytes = size_t(48) << 20;  // arrival counters, then the splits' partial results
constexpr size_t kTreeCounterBytes = 4096;                 // one uint32 per (row tile, key/value head)
constexpr int kTreeMaxSplits = 64;
// How the key splits are merged: by a second launch, or by the last
// workgroup of each tile to finish (arrival counters at the start of the
// workspace, zero between calls).
enum TreeMerge { kTreeMergeAuto = 0, kTreeMergeLaunch = 1, kTreeMergeLast = 2 };
// Key splits for (M, L, Hq, Hkv), the merge used (`merge` asks for one;
// one split needs none: kTreeMergeAuto comes back) and the workspace bytes
// they need; returns 0 (one split always fits: it writes the output
// directly), -1 if the tiles outnumber the counters.
int tree_attn_plan(int M, int L, int Hq, int Hkv, int merge, int* nsplit, int* merge_used, size_t* ws_bytes);
hipError_t launch_tree_attn(const uint16_t* q, const uint16_t* kc, const uint16_t* vc, const uint16_t* kd,
                            const uint16_t* vd, const uint64_t* masks, int M, int L, int Hq, int Hkv, float scale,
                            int merge, float* out, void* ws, hipStream_t stream);

}  // namespace w4
