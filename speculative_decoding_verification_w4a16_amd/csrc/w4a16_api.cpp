// C ABI of the W4A16 verify linear (declared in include/w4a16.h and
// include/w4a16_bench.h): argument validation, launch planning, the per-device
// split-K workspace, and dispatch to the kernels in w4a16_kernels.hip.
//
// Every check runs before the first HIP call, so a rejected call touches no
// device state; that is what lets the host tests exercise every error path
// without a GPU.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <map>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/w4_accept.h"
#include "../../include/w4_pass.h"
#include "../../include/w4_tree_attn.h"
#include "../../include/w4a16.h"
#include "../../include/w4a16_bench.h"
#include "w4_aux.h"
#include "w4_internal.h"

namespace {

constexpr int kMaxDevices = 64;

struct DeviceState {
    bool ready = false;
    w4::Workspace ws{};
    void* accept = nullptr;  // acceptance step workspace
    float* tree = nullptr;   // tree attention workspace
};

std::mutex g_mutex;
DeviceState g_dev[kMaxDevices];
thread_local char g_last_error[256] = "";

// Records the failing HIP call for w4_last_error and maps it to W4_ERR_HIP.
int hip_fail(const char* what, hipError_t e) {
    snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%d)", what, hipGetErrorName(e), (int)e);
    return W4_ERR_HIP;
}

int hip_status(const char* what, hipError_t e) { return e == hipSuccess ? W4_OK : hip_fail(what, e); }

// Workspaces and kernel attributes of the current device, created once.
int device_state(w4::Workspace* out, void** accept = nullptr, float** tree = nullptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail("hipGetDevice", e);
    if (dev < 0 || dev >= kMaxDevices) return hip_fail("device index", hipErrorInvalidDevice);
    std::lock_guard<std::mutex> lock(g_mutex);
    DeviceState& st = g_dev[dev];
    if (!st.ready) {
        e = w4::set_kernel_attributes();
        if (e != hipSuccess) return hip_fail("hipFuncSetAttribute", e);
        // all three workspaces or none (a failed call leaves nothing behind
        // and the next call tries again)
        void* part = nullptr;
        void* acc = nullptr;
        void* tree = nullptr;
        const char* what = "hipMalloc(workspace)";
        e = hipMalloc(&part, w4::kWorkspaceBytes);
        if (e == hipSuccess) {
            what = "hipMalloc(acceptance workspace)";
            e = hipMalloc(&acc, w4::kAcceptWorkspaceBytes);
        }
        if (e == hipSuccess) {
            what = "hipMalloc(tree attention workspace)";
            e = hipMalloc(&tree, w4::kTreeWorkspaceBytes);
        }
        if (e == hipSuccess) {
            // the tree attention's arrival counters start at zero; each call
            // leaves them at zero
            what = "hipMemset(tree attention counters)";
            e = hipMemset(tree, 0, w4::kTreeCounterBytes);
            if (e == hipSuccess) e = hipDeviceSynchronize();
        }
        if (e != hipSuccess) {
            if (part) (void)hipFree(part);
            if (acc) (void)hipFree(acc);
            if (tree) (void)hipFree(tree);
            return hip_fail(what, e);
        }
        st.ws.partial = (float*)part;
        st.ws.partial_bytes = w4::kWorkspaceBytes;
        st.accept = acc;
        st.tree = (float*)tree;
        st.ready = true;
    }
    if (out) *out = st.ws;
    if (accept) *accept = st.accept;
    if (tree) *tree = st.tree;
    return W4_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool draft_logits_ok(int sampled, const void* p) { return !sampled || p != nullptr; }

bool overlap(const void* a, size_t an, const void* b, size_t bn) {
    if (!a || !b || an == 0 || bn == 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + bn && b0 < a0 + an;
}

// Shape checks shared by every entry point.
int check_shape(int N, int K, int group) {
    if (N < 0 || K < 0) return W4_ERR_INVALID;
    if (group != w4::kGroup) return W4_ERR_UNSUPPORTED;
    if (N > W4_MAX_N || K > W4_MAX_K) return W4_ERR_UNSUPPORTED;
    if (K % w4::kGroup != 0 || N % 8 != 0) return W4_ERR_UNSUPPORTED;
    return W4_OK;
}

size_t chunks(int N) { return ((size_t)N + w4::kChunkN - 1) / w4::kChunkN; }

void tile_sizes(int N, int K, size_t* qb, size_t* sb, size_t* zb) {
    const size_t npad = chunks(N) * w4::kChunkN;
    *qb = npad * (size_t)K / 2;
    *sb = npad * (size_t)(K / w4::kGroup) * 2;
    *zb = npad * (size_t)(K / w4::kGroup) / 2;
}

// Validation of one linear call; fills the plan on success.
int check_linear(const uint16_t* x, const uint32_t* qt, const uint16_t* st, const uint16_t* zt, int M, int N, int K,
                 int group, const void* y, int out_dtype, int kernel, int splits, int kwaves, w4::Plan* plan) {
    if (M < 0) return W4_ERR_INVALID;
    int rc = check_shape(N, K, group);
    if (rc != W4_OK) return rc;
    if (M > W4_MAX_M) return W4_ERR_UNSUPPORTED;
    if (kernel < W4_KERNEL_AUTO || kernel > W4_KERNEL_MFMA || splits < 0) return W4_ERR_INVALID;
    if (kwaves < 0) return W4_ERR_INVALID;
    if (out_dtype != W4_OUT_F32 && out_dtype != W4_OUT_BF16) return W4_ERR_INVALID;
    if (kernel == W4_KERNEL_GEMV && M > 1) return W4_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return W4_OK;  // nothing to compute
    if (!y) return W4_ERR_INVALID;
    if (!aligned(y, 16)) return W4_ERR_INVALID;
    const size_t ybytes = (size_t)M * N * (out_dtype == W4_OUT_BF16 ? 2 : 4);
    if (K == 0) return W4_OK;  // y = 0
    if (!x || !qt || !st || !zt) return W4_ERR_INVALID;
    if (!aligned(x, 16) || !aligned(qt, 16) || !aligned(st, 8) || !aligned(zt, 2)) return W4_ERR_INVALID;
    size_t qb, sb, zb;
    tile_sizes(N, K, &qb, &sb, &zb);
    if (overlap(y, ybytes, x, (size_t)M * K * 2) || overlap(y, ybytes, qt, qb) || overlap(y, ybytes, st, sb) ||
        overlap(y, ybytes, zt, zb))
        return W4_ERR_INVALID;
    if (plan) {
        if (w4::plan_linear(M, N, K, kernel, splits, kwaves, w4::kWorkspaceBytes, plan) != 0)
            return W4_ERR_UNSUPPORTED;
    }
    return W4_OK;
}

// The split-K partials' bytes of a plan.
size_t partial_bytes(const w4::Plan& plan, int M, int N) {
    return plan.splits > 1 ? (size_t)plan.splits * M * chunks(N) * w4::kChunkN * sizeof(float) : 0;
}

int run_linear(const uint16_t* x, const uint32_t* qt, const uint16_t* st, const uint16_t* zt, int M, int N, int K,
               void* y, int out_dtype, const w4::Plan& plan, hipStream_t stream) {
    if (M == 0 || N == 0) return W4_OK;
    if (K == 0) {
        // y = 0: M*N fp32 zeros, or half as many bytes of bf16 zeros
        const size_t n = (size_t)M * N / (out_dtype == W4_OUT_BF16 ? 2 : 1);
        return hip_status("zero_kernel launch", w4::launch_zero((float*)y, n, stream));
    }
    w4::Workspace ws{};
    if (plan.splits > 1) {
        int rc = device_state(&ws);
        if (rc != W4_OK) return rc;
    } else {
        int rc = device_state(nullptr);  // kernel attributes
        if (rc != W4_OK) return rc;
    }
    return hip_status("verify-linear launch", w4::launch_linear(plan, x, qt, st, zt, M, N, K, y,
                                                                out_dtype == W4_OUT_BF16, ws, stream));
}

}  // namespace

extern "C" {

const char* w4_status_str(int status) {
    switch (status) {
        case W4_OK: return "W4_OK";
        case W4_ERR_INVALID: return "W4_ERR_INVALID: invalid argument (null, negative, misaligned or overlapping)";
        case W4_ERR_UNSUPPORTED: return "W4_ERR_UNSUPPORTED: unsupported shape or group size";
        case W4_ERR_HIP: return "W4_ERR_HIP: a HIP runtime call failed";
        case W4_ERR_TIMEOUT: return "W4_ERR_TIMEOUT: a verify pass waited too long for a producer (results invalid)";
        default: return "W4_ERR_UNKNOWN: unknown status code";
    }
}

const char* w4_last_error(void) { return g_last_error; }

int w4_init(void) { return device_state(nullptr); }

int w4_repacked_sizes(int N, int K, int group, size_t* qweight_bytes, size_t* scales_bytes, size_t* zeros_bytes) {
    if (!qweight_bytes || !scales_bytes || !zeros_bytes) return W4_ERR_INVALID;
    int rc = check_shape(N, K, group);
    if (rc != W4_OK) return rc;
    tile_sizes(N, K, qweight_bytes, scales_bytes, zeros_bytes);
    return W4_OK;
}

int w4_repack(const int32_t* qweight, const uint16_t* scales, const int32_t* zeros, int N, int K, int group,
              uint32_t* qweight_t, uint16_t* scales_t, uint16_t* zeros_t, void* stream) {
    int rc = check_shape(N, K, group);
    if (rc != W4_OK) return rc;
    if (N == 0 || K == 0) return W4_OK;
    if (!qweight || !scales || !zeros || !qweight_t || !scales_t || !zeros_t) return W4_ERR_INVALID;
    if (!aligned(qweight, 4) || !aligned(scales, 2) || !aligned(zeros, 4) || !aligned(qweight_t, 16) ||
        !aligned(scales_t, 8) || !aligned(zeros_t, 2))
        return W4_ERR_INVALID;
    size_t qb, sb, zb;
    tile_sizes(N, K, &qb, &sb, &zb);
    const size_t cq = (size_t)N * K / 2, cs = (size_t)N * (K / w4::kGroup) * 2, cz = cs / 4;
    const void* ins[3] = {qweight, scales, zeros};
    const size_t inb[3] = {cq, cs, cz};
    const void* outs[3] = {qweight_t, scales_t, zeros_t};
    const size_t outb[3] = {qb, sb, zb};
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j) {
            if (overlap(outs[i], outb[i], ins[j], inb[j])) return W4_ERR_INVALID;
            if (i != j && overlap(outs[i], outb[i], outs[j], outb[j])) return W4_ERR_INVALID;
        }
    return hip_status("repack launch", w4::launch_repack(qweight, scales, zeros, N, K, qweight_t, scales_t, zeros_t,
                                                          (hipStream_t)stream));
}

int w4a16_linear_tune(const uint16_t* x, const uint32_t* qweight_t, const uint16_t* scales_t,
                      const uint16_t* zeros_t, int M, int N, int K, int group, void* y, int out_dtype, int kernel,
                      int splits, int kwaves, void* stream) {
    w4::Plan plan{};
    int rc =
        check_linear(x, qweight_t, scales_t, zeros_t, M, N, K, group, y, out_dtype, kernel, splits, kwaves, &plan);
    if (rc != W4_OK) return rc;
    return run_linear(x, qweight_t, scales_t, zeros_t, M, N, K, y, out_dtype, plan, (hipStream_t)stream);
}

int w4a16_linear_out(const uint16_t* x, const uint32_t* qweight_t, const uint16_t* scales_t,
                     const uint16_t* zeros_t, int M, int N, int K, int group, void* y, int out_dtype, int kernel,
                     int splits, void* stream) {
    return w4a16_linear_tune(x, qweight_t, scales_t, zeros_t, M, N, K, group, y, out_dtype, kernel, splits, 0,
                             stream);
}

int w4a16_linear_out_noalloc(const uint16_t* x, const uint32_t* qweight_t, const uint16_t* scales_t,
                             const uint16_t* zeros_t, int M, int N, int K, int group, void* y, int out_dtype,
                             int kernel, int splits, void* stream) {
    w4::Plan plan{};
    int rc = check_linear(x, qweight_t, scales_t, zeros_t, M, N, K, group, y, out_dtype, kernel, splits, 0, &plan);
    if (rc != W4_OK) return rc;
    if (M == 0 || N == 0) return W4_OK;
    // a forced split count whose partials would not fit the scratch is
    // refused (the planner would otherwise lower it): the caller asked for a
    // decomposition this entry point cannot hold
    if (splits > 0 && plan.splits < std::min(splits, K / w4::kGroup) &&
        (size_t)std::min(splits, K / w4::kGroup) * M * chunks(N) * w4::kChunkN * sizeof(float) >
            w4::kNoAllocScratchBytes)
        return W4_ERR_UNSUPPORTED;
    if (partial_bytes(plan, M, N) > w4::kNoAllocScratchBytes) return W4_ERR_UNSUPPORTED;
    if (K == 0) {
        const size_t n = (size_t)M * N / (out_dtype == W4_OUT_BF16 ? 2 : 1);
        return hip_status("zero_kernel launch", w4::launch_zero((float*)y, n, (hipStream_t)stream));
    }
    w4::Workspace ws{};
    hipError_t e = w4::noalloc_scratch(&ws);
    if (e != hipSuccess) return hip_fail("hipGetSymbolAddress(scratch)", e);
    return hip_status("verify-linear launch", w4::launch_linear(plan, x, qweight_t, scales_t, zeros_t, M, N, K, y,
                                                                out_dtype == W4_OUT_BF16, ws,
                                                                (hipStream_t)stream));
}

int w4a16_linear_cfg(const uint16_t* x, const uint32_t* qweight_t, const uint16_t* scales_t,
                     const uint16_t* zeros_t, int M, int N, int K, int group, float* y, int kernel, int splits,
                     void* stream) {
    return w4a16_linear_out(x, qweight_t, scales_t, zeros_t, M, N, K, group, y, W4_OUT_F32, kernel, splits,
                            stream);
}

int w4a16_linear(const uint16_t* x, const uint32_t* qweight_t, const uint16_t* scales_t, const uint16_t* zeros_t,
                 int M, int N, int K, int group, float* y, void* stream) {
    return w4a16_linear_cfg(x, qweight_t, scales_t, zeros_t, M, N, K, group, y, W4_KERNEL_AUTO, 0, stream);
}

int w4a16_plan(int M, int N, int K, int group, int kernel, int splits, int kwaves, int* kernel_out,
               int* splits_out, int* kwaves_out, int* grid_out, int* block_out, int* lds_out) {
    if (M <= 0 || N <= 0 || K <= 0) return W4_ERR_INVALID;
    int rc = check_shape(N, K, group);
    if (rc != W4_OK) return rc;
    if (M > W4_MAX_M) return W4_ERR_UNSUPPORTED;
    if (kernel < W4_KERNEL_AUTO || kernel > W4_KERNEL_MFMA || splits < 0 || kwaves < 0) return W4_ERR_INVALID;
    if (kernel == W4_KERNEL_GEMV && M > 1) return W4_ERR_UNSUPPORTED;
    w4::Plan p{};
    if (w4::plan_linear(M, N, K, kernel, splits, kwaves, w4::kWorkspaceBytes, &p) != 0) return W4_ERR_UNSUPPORTED;
    if (kernel_out) *kernel_out = p.kernel;
    if (splits_out) *splits_out = p.splits;
    if (kwaves_out) *kwaves_out = p.kw;
    if (grid_out) *grid_out = p.grid;
    if (block_out) *block_out = p.block;
    if (lds_out) *lds_out = p.lds;
    return W4_OK;
}

int w4a16_verify_pass(const w4_linear_desc* linears, int n, int M, int group, void* stream) {
    if (n < 0 || (n > 0 && !linears)) return W4_ERR_INVALID;
    // validate everything first so a bad entry launches nothing
    for (int i = 0; i < n; ++i) {
        const w4_linear_desc& d = linears[i];
        int rc = check_linear(d.x, d.qweight_t, d.scales_t, d.zeros_t, M, d.N, d.K, group, d.y, W4_OUT_F32,
                              W4_KERNEL_AUTO, 0, 0, nullptr);
        if (rc != W4_OK) return rc;
    }
    for (int i = 0; i < n; ++i) {
        const w4_linear_desc& d = linears[i];
        w4::Plan plan{};
        if (M > 0 && d.N > 0 && d.K > 0 &&
            w4::plan_linear(M, d.N, d.K, W4_KERNEL_AUTO, 0, 0, w4::kWorkspaceBytes, &plan) != 0)
            return W4_ERR_UNSUPPORTED;
        int rc = run_linear(d.x, d.qweight_t, d.scales_t, d.zeros_t, M, d.N, d.K, d.y, W4_OUT_F32, plan,
                            (hipStream_t)stream);
        if (rc != W4_OK) return rc;
    }
    return W4_OK;
}

int w4_unpack(const uint32_t* qweight_t, const uint16_t* zeros_t, int N, int K, int group, uint8_t* q_out,
              uint8_t* z_out, void* stream) {
    int rc = check_shape(N, K, group);
    if (rc != W4_OK) return rc;
    if (N == 0 || K == 0) return W4_OK;
    if (!qweight_t || !zeros_t || !q_out || !z_out) return W4_ERR_INVALID;
    if (!aligned(qweight_t, 16) || !aligned(zeros_t, 2)) return W4_ERR_INVALID;
    return hip_status("unpack launch", w4::launch_unpack(qweight_t, zeros_t, N, K, q_out, z_out, (hipStream_t)stream));
}

int w4_bench_read_blocks(void) { return w4::kBenchReadBlocks; }

int w4_bench_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
    if (!buf || !sink || bytes % 16 != 0 || !aligned(buf, 16) || !aligned(sink, 4)) return W4_ERR_INVALID;
    if (bytes == 0) return W4_OK;
    return hip_status("bench_read launch",
                      w4::launch_bench_read(buf, bytes, sink, w4::kBenchReadBlocks, (hipStream_t)stream));
}

int w4_bench_copy(void* dst, const void* src, size_t bytes, void* stream) {
    if (!dst || !src || bytes % 16 != 0 || !aligned(dst, 16) || !aligned(src, 16)) return W4_ERR_INVALID;
    if (overlap(dst, bytes, src, bytes)) return W4_ERR_INVALID;
    if (bytes == 0) return W4_OK;
    return hip_status("bench_copy launch", w4::launch_bench_copy(dst, src, bytes, (hipStream_t)stream));
}

}  // extern "C"

namespace {

int accept_call(const float* logits, const float* draft_logits, const int32_t* draft, const float* u, int K, int V,
                int sampled, int32_t* out, void* stream) {
    if (K < 0 || V < 0) return W4_ERR_INVALID;
    if (K > W4_ACCEPT_MAX_K || V > W4_ACCEPT_MAX_V || V % 4 != 0) return W4_ERR_UNSUPPORTED;
    if (V < 4) return W4_ERR_UNSUPPORTED;
    if (!logits || !draft_logits_ok(sampled, draft_logits) || !out || (K > 0 && !draft) || (sampled && !u))
        return W4_ERR_INVALID;
    if (!aligned(logits, 16) || (sampled && !aligned(draft_logits, 16)) || !aligned(out, 4) ||
        (K > 0 && !aligned(draft, 4)) || (sampled && !aligned(u, 4)))
        return W4_ERR_INVALID;
    const size_t lb = (size_t)(K + 1) * V * 4, db = sampled ? (size_t)K * V * 4 : 0;
    if (overlap(out, 8, logits, lb) || overlap(out, 8, draft_logits, db) || overlap(out, 8, draft, (size_t)K * 4) ||
        (sampled && overlap(out, 8, u, (size_t)(K + 1) * 4)))
        return W4_ERR_INVALID;
    if (w4::accept_workspace_bytes(K, V) > w4::kAcceptWorkspaceBytes) return W4_ERR_UNSUPPORTED;
    void* ws = nullptr;
    int rc = device_state(nullptr, &ws);
    if (rc != W4_OK) return rc;
    return hip_status("acceptance launch", w4::launch_accept(logits, sampled ? draft_logits : logits, draft, u, K, V,
                                                             sampled, out, ws, (hipStream_t)stream));
}

}  // namespace

extern "C" {

int w4_accept_greedy(const float* logits, const int32_t* draft, int K, int V, int32_t* out, void* stream) {
    return accept_call(logits, nullptr, draft, nullptr, K, V, 0, out, stream);
}

int w4_accept_sample(const float* logits, const float* draft_logits, const int32_t* draft, const float* u, int K,
                     int V, int32_t* out, void* stream) {
    return accept_call(logits, draft_logits, draft, u, K, V, 1, out, stream);
}

}

static_assert(W4_TREE_MERGE_AUTO == w4::kTreeMergeAuto && W4_TREE_MERGE_LAUNCH == w4::kTreeMergeLaunch &&
                  W4_TREE_MERGE_LAST == w4::kTreeMergeLast,
              "merge choices");

extern "C" int w4_tree_attention_plan(int M, int L, int num_heads, int num_kv_heads, int merge, int* splits,
                                      int* merge_used) {
    if (M < 1 || L < 0 || num_heads <= 0 || num_kv_heads <= 0) return W4_ERR_INVALID;
    if (merge < W4_TREE_MERGE_AUTO || merge > W4_TREE_MERGE_LAST) return W4_ERR_INVALID;
    if (M > W4_TREE_MAX_M || L > W4_TREE_MAX_L || num_heads % num_kv_heads != 0 || num_heads > 256)
        return W4_ERR_UNSUPPORTED;
    int s = 0, used = 0;
    if (w4::tree_attn_plan(M, L, num_heads, num_kv_heads, merge, &s, &used, nullptr) != 0) return W4_ERR_UNSUPPORTED;
    if (splits) *splits = s;
    if (merge_used) *merge_used = used;
    return W4_OK;
}

extern "C" int w4_tree_attention(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                                 const uint16_t* k_draft, const uint16_t* v_draft, const uint64_t* masks, int M,
                                 int L, int num_heads, int num_kv_heads, int head_dim, float scale, float* out,
                                 void* stream) {
    return w4_tree_attention_ex(q, k_cache, v_cache, k_draft, v_draft, masks, M, L, num_heads, num_kv_heads,
                                head_dim, scale, W4_TREE_MERGE_AUTO, out, stream);
}

extern "C" int w4_tree_attention_ex(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                                    const uint16_t* k_draft, const uint16_t* v_draft, const uint64_t* masks, int M,
                                    int L, int num_heads, int num_kv_heads, int head_dim, float scale, int merge,
                                    float* out, void* stream) {
    if (M < 0 || L < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0) return W4_ERR_INVALID;
    if (merge < W4_TREE_MERGE_AUTO || merge > W4_TREE_MERGE_LAST) return W4_ERR_INVALID;
    if (!(scale >= 0.0f) || scale > 1e30f) return W4_ERR_INVALID;  // rejects NaN
    if (head_dim != w4::kTreeHeadDim || M > W4_TREE_MAX_M || L > W4_TREE_MAX_L || num_heads % num_kv_heads != 0 ||
        num_heads > 256)
        return W4_ERR_UNSUPPORTED;
    if (M == 0) return W4_OK;
    if (!q || !k_draft || !v_draft || !masks || !out || (L > 0 && (!k_cache || !v_cache))) return W4_ERR_INVALID;
    if (!aligned(q, 16) || !aligned(k_draft, 16) || !aligned(v_draft, 16) || !aligned(masks, 8) || !aligned(out, 16) ||
        (L > 0 && (!aligned(k_cache, 16) || !aligned(v_cache, 16))))
        return W4_ERR_INVALID;
    const size_t ob = (size_t)M * num_heads * head_dim * 4;
    const size_t qb = (size_t)M * num_heads * head_dim * 2, cb = (size_t)L * num_kv_heads * head_dim * 2,
                 db = (size_t)M * num_kv_heads * head_dim * 2;
    if (overlap(out, ob, q, qb) || overlap(out, ob, k_cache, cb) || overlap(out, ob, v_cache, cb) ||
        overlap(out, ob, k_draft, db) || overlap(out, ob, v_draft, db) || overlap(out, ob, masks, (size_t)M * 8))
        return W4_ERR_INVALID;
    if (w4::tree_attn_plan(M, L, num_heads, num_kv_heads, merge, nullptr, nullptr, nullptr) != 0)
        return W4_ERR_UNSUPPORTED;
    float* ws = nullptr;
    int rc = device_state(nullptr, nullptr, &ws);
    if (rc != W4_OK) return rc;
    const float sc = scale > 0.0f ? scale : 1.0f / sqrtf((float)head_dim);
    return hip_status("tree attention launch",
                      w4::launch_tree_attn(q, k_cache, v_cache, k_draft, v_draft, masks, M, L, num_heads,
                                           num_kv_heads, sc, merge, out, ws, (hipStream_t)stream));
}

// ---------------------------------------------------------------------------
// the verify pass as one launch (include/w4_pass.h)
// ---------------------------------------------------------------------------

struct w4_pass {
    int device = 0;
    int n = 0, M = 0, U = 0, grid = 0;
    bool persistent = false;
    w4::PassLinear* tab = nullptr;  // device table of the linears
    uint32_t* counters = nullptr;   // device: chunks done per linear (sub-counters), split chunks' arrivals,
                                    // exited workgroups, error flag
    int arrivals = 0;               // split chunks (K-split units' arrival counters)
    float* part = nullptr;          // device: partial tiles of the K-split units
    std::vector<w4_pass_linear> lin;
    std::vector<w4::Plan> plans;    // per-linear launches (M > kPassMaxM)
    w4::Workspace ws{};
    uint32_t spin_limit = 1u << 24; // polls (each about 50 ns apart) before a wait gives up
};

namespace {

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

std::vector<int> sorted_deps(const w4_pass_linear& d) {
    std::vector<int> v(d.deps, d.deps + d.ndeps);
    std::sort(v.begin(), v.end());
    return v;
}

Range range_of(const void* p, size_t bytes) { return Range{(uintptr_t)p, (uintptr_t)p + bytes}; }
Range lines_of(Range r) { return Range{r.lo & ~(uintptr_t)127, (r.hi + 127) & ~(uintptr_t)127}; }
bool meets(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo < a.hi && b.lo < b.hi; }

// Per-linear argument checks of a pass entry.
// Elements between rows of a pass linear's x (0 means K).
int pass_ldx(const w4_pass_linear& d) { return d.ldx == 0 ? d.K : d.ldx; }

// Bytes from x to the end of row M - 1's K values.
size_t pass_x_bytes(const w4_pass_linear& d, int M) {
    return M > 0 ? ((size_t)(M - 1) * pass_ldx(d) + d.K) * 2 : 0;
}

int check_pass_linear(const w4_pass_linear& d, int i, int M, int group) {
    if (d.N < 0 || d.K < 0 || d.ndeps < 0) return W4_ERR_INVALID;
    if (d.ldx != 0 && (d.ldx < d.K || d.ldx % 8 != 0)) return W4_ERR_INVALID;
    int rc = check_shape(d.N, d.K, group);
    if (rc != W4_OK) return rc;
    if (d.N < 8 || d.K < w4::kGroup || d.ndeps > W4_PASS_MAX_DEPS) return W4_ERR_UNSUPPORTED;
    if (!d.y && !d.y_bf16) return W4_ERR_INVALID;
    if (!std::isfinite(d.alpha)) return W4_ERR_INVALID;
    if ((d.y && !aligned(d.y, 128)) || (d.y_bf16 && !aligned(d.y_bf16, 128))) return W4_ERR_INVALID;
    if (!aligned(d.zeros_t, 4)) return W4_ERR_INVALID;  // the pass kernel reads zero records in aligned pairs
    for (int j = 0; j < d.ndeps; ++j) {
        if (d.deps[j] < 0 || d.deps[j] >= i) return W4_ERR_INVALID;
        for (int k = 0; k < j; ++k)
            if (d.deps[k] == d.deps[j]) return W4_ERR_INVALID;
    }
    if (M == 0) return W4_OK;
    if (d.y) {
        rc = check_linear(d.x, d.qweight_t, d.scales_t, d.zeros_t, M, d.N, d.K, group, d.y, W4_OUT_F32,
                          W4_KERNEL_AUTO, 0, 0, nullptr);
        if (rc != W4_OK) return rc;
    }
    if (d.y_bf16) {
        rc = check_linear(d.x, d.qweight_t, d.scales_t, d.zeros_t, M, d.N, d.K, group, d.y_bf16, W4_OUT_BF16,
                          W4_KERNEL_AUTO, 0, 0, nullptr);
        if (rc != W4_OK) return rc;
    }
    // the outputs may not overlap the whole span of a strided x either
    const size_t xb = pass_x_bytes(d, M);
    if (overlap(d.y, (size_t)M * d.N * 4, d.x, xb) || overlap(d.y_bf16, (size_t)M * d.N * 2, d.x, xb))
        return W4_ERR_INVALID;
    return W4_OK;
}

// Hazards between the linears of a pass (see w4_pass_create).
// The ranges of a pass, swept in address order: every pair of ranges whose
// 128-byte lines meet is classified (outputs against outputs, weights and
// inputs; inputs and weights may share lines with each other), so the check
// takes O(n log n) plus the pairs that do meet, not a comparison of every
// output with every other range.
int check_pass_hazards(const w4_pass_linear* L, int n, int M) {
    enum Kind { kOut, kWeight, kIn };
    struct Item {
        Range r, lines;  // exact bytes, and rounded out to whole 128-byte lines
        Kind kind;
        int owner;       // the linear
    };
    std::vector<Item> items;
    items.reserve((size_t)n * 6);
    auto add = [&](Range r, Kind k, int i) {
        if (r.lo < r.hi) items.push_back(Item{r, lines_of(r), k, i});
    };
    for (int i = 0; i < n; ++i) {
        const w4_pass_linear& d = L[i];
        size_t qb, sb, zb;
        tile_sizes(d.N, d.K, &qb, &sb, &zb);
        add(range_of(d.x, pass_x_bytes(d, M)), kIn, i);
        add(range_of(d.qweight_t, qb), kWeight, i);
        add(range_of(d.scales_t, sb), kWeight, i);
        add(range_of(d.zeros_t, zb), kWeight, i);
        if (d.y) add(range_of(d.y, (size_t)M * d.N * 4), kOut, i);
        if (d.y_bf16) add(range_of(d.y_bf16, (size_t)M * d.N * 2), kOut, i);
    }
    std::sort(items.begin(), items.end(), [](const Item& a, const Item& b) { return a.lines.lo < b.lines.lo; });
    // a pair whose lines meet: an output may meet only the inputs of its
    // consumers (exactly, listed, later), never another output, weights or a
    // line of any other input
    auto pair_ok = [&](const Item& a, const Item& b) {
        if (a.kind != kOut && b.kind != kOut) return true;
        if (a.kind == kOut && b.kind == kOut) return false;
        const Item& o = a.kind == kOut ? a : b;
        const Item& x = a.kind == kOut ? b : a;
        if (x.kind == kWeight) return false;
        if (!meets(o.r, x.r)) return false;  // an unrelated input shares a cache line with the output
        const int i = x.owner, j = o.owner;  // linear i reads linear j's output
        if (i <= j) return false;
        for (int k = 0; k < L[i].ndeps; ++k)
            if (L[i].deps[k] == j) return true;
        return false;
    };
    std::vector<size_t> active;  // items whose lines may still meet later ones
    for (size_t b = 0; b < items.size(); ++b) {
        size_t keep = 0;
        for (size_t a : active) {
            if (items[a].lines.hi <= items[b].lines.lo) continue;  // ends before b starts: done
            if (!pair_ok(items[a], items[b])) return W4_ERR_INVALID;
            active[keep++] = a;
        }
        active.resize(keep);
        active.push_back(b);
    }
    return W4_OK;
}

void pass_free(w4_pass* p) {
    if (!p) return;
    if (p->tab) (void)hipFree(p->tab);
    if (p->counters) (void)hipFree(p->counters);
    if (p->part) (void)hipFree(p->part);
    delete p;
}

}  // namespace

extern "C" {

int w4_pass_create(const w4_pass_linear* linears, int n, int M, int group, w4_pass** out) {
    return w4_pass_create_mode(linears, n, M, group, W4_PASS_AUTO, out);
}

int w4_pass_create_mode(const w4_pass_linear* linears, int n, int M, int group, int mode, w4_pass** out) {
    if (!out) return W4_ERR_INVALID;
    *out = nullptr;
    if (n < 0 || M < 0 || (n > 0 && !linears)) return W4_ERR_INVALID;
    if (mode != W4_PASS_AUTO && mode != W4_PASS_PERSISTENT && mode != W4_PASS_LAUNCHES) return W4_ERR_INVALID;
    if (group != w4::kGroup || M > W4_MAX_M || n > W4_PASS_MAX_LINEARS) return W4_ERR_UNSUPPORTED;
    if (mode == W4_PASS_PERSISTENT && M > w4::kPassMaxM) return W4_ERR_UNSUPPORTED;
    for (int i = 0; i < n; ++i) {
        int rc = check_pass_linear(linears[i], i, M, group);
        if (rc != W4_OK) return rc;
    }
    if (M > 0) {
        int rc = check_pass_hazards(linears, n, M);
        if (rc != W4_OK) return rc;
    }
    w4_pass* p = new (std::nothrow) w4_pass();
    if (!p) return W4_ERR_HIP;
    p->n = n;
    p->M = M;
    p->lin.assign(linears, linears + n);
    // the persistent kernel is possible at M <= kPassMaxM; whether it is
    // chosen is decided once the dependency classes are known
    p->persistent = M >= 1 && M <= w4::kPassMaxM && mode != W4_PASS_LAUNCHES;
    hipError_t e = hipGetDevice(&p->device);
    if (e != hipSuccess) {
        pass_free(p);
        return hip_fail("hipGetDevice", e);
    }
    int cus = 0;
    if (p->persistent && n > 0) {
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, p->device);
        if (e != hipSuccess) {
            pass_free(p);
            return hip_fail("hipDeviceGetAttribute", e);
        }
    }
    std::vector<w4::PassLinear> tab(n);
    std::map<std::vector<int>, int> first_with;  // a set of producers -> the first linear that has it
    int U = 0, arrivals = 0;
    size_t tiles = 0;
    for (int i = 0; i < n; ++i) {
        const w4_pass_linear& d = linears[i];
        w4::PassLinear& t = tab[i];
        t.x = d.x;
        t.qt = d.qweight_t;
        t.st = d.scales_t;
        t.zt = d.zeros_t;
        t.y = d.y;
        t.yb = d.y_bf16;
        t.alpha = d.alpha;
        t.N = d.N;
        t.K = d.K;
        t.ldx = pass_ldx(d);
        t.NC = (int)chunks(d.N);
        t.G = d.K / w4::kGroup;
        t.S = 1;
        t.gps = t.G;
        t.kw = std::min(w4::kPassWaves, t.G);
        t.ndep = d.ndeps;
        for (int j = 0; j < w4::kPassMaxDeps; ++j) {
            t.dep[j] = j < d.ndeps ? d.deps[j] : 0;
            t.dep_units[j] = j < d.ndeps ? (int)chunks(linears[d.deps[j]].N) : 0;
        }
        // linears with the same set of producers share a class: once one
        // has seen its producers complete, the others need not wait
        t.dep_class = -1;
        if (d.ndeps > 0) t.dep_class = first_with.emplace(sorted_deps(d), i).first->second;
    }
    // Which form (W4_PASS_AUTO).  The persistent kernel pays, at each
    // dependency class, the wait for its producers' last units and a memory
    // round trip before the first multiply-add; per-linear launches pay a
    // launch gap per linear and run the linears of a class one after the
    // other.  Measured on MI355X over the 80-layer Llama-3-70B pass (M = 1 /
    // M = 5): with q, k, v and gate, up as separate linears (561 linears in
    // 321 classes) the persistent kernel takes 7.6 / 8.6 ms against 8.9 /
    // 9.8 for launches; with q|k|v and gate|up fused (321 linears, one per
    // class) 7.6 / 8.6 against 7.1 / 7.8.  So the persistent kernel is chosen
    // when the classes hold at least 1.25 linears on average.
    if (p->persistent && mode == W4_PASS_AUTO) {
        long classes = 0;
        bool free_class = false;  // linears without producers form one class
        for (int i = 0; i < n; ++i) {
            if (tab[i].dep_class < 0) free_class = true;
            else if (tab[i].dep_class == i) ++classes;
        }
        classes += free_class ? 1 : 0;
        p->persistent = 4L * n >= 5L * classes;
    }
    // K slices.  The linears of one dependency class run side by side, and
    // their consumers wait for all of them; when together they have fewer
    // chunks than half the CUs, the other CUs would sit idle.  Their chunks
    // are then split into S slices of K (S units each), as long as a slice
    // keeps every wave of a workgroup busy for two rounds (measured: q and o
    // in two slices of four waves each made the pass slower).  The last
    // slice of a chunk to finish adds the slices' partial tiles in slice
    // order.
    if (p->persistent) {
        // (the linears without producers form one class, index n)
        std::vector<long> class_chunks(n + 1, 0);
        for (int i = 0; i < n; ++i) class_chunks[tab[i].dep_class >= 0 ? tab[i].dep_class : n] += tab[i].NC;
        const int per_wave = 2 * w4::kPassRing;  // groups of two rounds
        for (int i = 0; i < n; ++i) {
            w4::PassLinear& t = tab[i];
            const long cc = class_chunks[t.dep_class >= 0 ? t.dep_class : n];
            const int s_cus = (int)std::max<long>(1, cus / std::max<long>(cc, 1));
            const int s_k = std::max(1, t.G / (w4::kPassWaves * per_wave));
            int S = std::min(s_cus, s_k);
            if (S > 1) {
                t.gps = (t.G + S - 1) / S;
                t.S = (t.G + t.gps - 1) / t.gps;
                t.kw = std::max(1, std::min(w4::kPassWaves, (t.G - (t.S - 1) * t.gps) / per_wave));
            }
        }
    }
    for (int i = 0; i < n; ++i) {
        w4::PassLinear& t = tab[i];
        t.unit0 = U;
        t.part0 = t.S > 1 ? (int)tiles : 0;
        t.arr0 = t.S > 1 ? arrivals : 0;
        if (t.S > 1) {
            tiles += (size_t)t.NC * t.S;
            arrivals += t.NC;
        }
        U += t.NC * t.S;
    }
    p->U = U;
    p->arrivals = arrivals;
    if (p->persistent && n > 0) {
        int per_cu = 0;
        e = w4::pass_occupancy(M, &per_cu);
        if (e != hipSuccess || per_cu < 1) {
            pass_free(p);
            return hip_fail("pass occupancy", e != hipSuccess ? e : hipErrorInvalidConfiguration);
        }
        p->grid = std::max(1, std::min(U, cus));
        e = hipMalloc((void**)&p->tab, sizeof(w4::PassLinear) * n);
        const size_t words = w4::pass_counter_words(n, arrivals);
        if (e == hipSuccess) e = hipMalloc((void**)&p->counters, sizeof(uint32_t) * words);
        if (e == hipSuccess && tiles > 0)
            e = hipMalloc((void**)&p->part, sizeof(float) * tiles * w4::pass_tile_floats(M));
        if (e == hipSuccess) e = hipMemcpy(p->tab, tab.data(), sizeof(w4::PassLinear) * n, hipMemcpyHostToDevice);
        if (e == hipSuccess) e = hipMemset(p->counters, 0, sizeof(uint32_t) * words);
        if (e == hipSuccess) e = hipDeviceSynchronize();
        if (e != hipSuccess) {
            pass_free(p);
            return hip_fail("pass set-up", e);
        }
    } else if (M > 0) {
        // per-linear launches: their plans, and the split-K workspace now
        p->plans.resize(n);
        for (int i = 0; i < n; ++i)
            if (w4::plan_linear(M, linears[i].N, linears[i].K, W4_KERNEL_AUTO, 0, 0, w4::kWorkspaceBytes,
                                &p->plans[i]) != 0) {
                pass_free(p);
                return W4_ERR_UNSUPPORTED;
            }
        int rc = device_state(&p->ws);
        if (rc != W4_OK) {
            pass_free(p);
            return rc;
        }
    }
    *out = p;
    return W4_OK;
}

int w4_pass_run(w4_pass* p, void* stream) {
    if (!p) return W4_ERR_INVALID;
    if (p->M == 0 || p->n == 0) return W4_OK;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail("hipGetDevice", e);
    if (dev != p->device) return W4_ERR_INVALID;
    if (p->persistent) {
        w4::PassLaunch l;
        l.tab = p->tab;
        l.n = p->n;
        l.U = p->U;
        l.M = p->M;
        l.done = p->counters;
        l.arrivals = p->arrivals;
        l.state = p->counters + w4::pass_counter_words(p->n, p->arrivals) - 2;
        l.part = p->part;
        l.spin_limit = p->spin_limit;
        l.grid = p->grid;
        return hip_status("pass launch", w4::launch_pass(l, (hipStream_t)stream));
    }
    for (int i = 0; i < p->n; ++i) {
        const w4_pass_linear& d = p->lin[i];
        e = w4::launch_linear_io(p->plans[i], d.x, pass_ldx(d), d.qweight_t, d.scales_t, d.zeros_t, p->M, d.N, d.K, d.y,
                                 d.y_bf16, d.alpha, p->ws, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail("pass linear launch", e);
    }
    return W4_OK;
}

int w4_pass_check(w4_pass* p, void* stream) {
    if (!p) return W4_ERR_INVALID;
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return hip_fail("hipStreamSynchronize", e);
    if (!p->persistent || !p->counters) return W4_OK;
    uint32_t flag = 0;
    uint32_t* const err = p->counters + w4::pass_counter_words(p->n, p->arrivals) - 1;
    e = hipMemcpy(&flag, err, sizeof(flag), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail("hipMemcpy(pass flag)", e);
    if (flag == 0) return W4_OK;
    e = hipMemset(err, 0, sizeof(uint32_t));
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail("hipMemset(pass flag)", e);
    return W4_ERR_TIMEOUT;
}

int w4_pass_info(const w4_pass* p, int* persistent, int* grid, int* units) {
    if (!p) return W4_ERR_INVALID;
    if (persistent) *persistent = p->persistent ? 1 : 0;
    if (grid) *grid = p->grid;
    if (units) *units = p->U;
    return W4_OK;
}

int w4_pass_set_spin_limit(w4_pass* p, uint32_t polls) {
    if (!p) return W4_ERR_INVALID;
    p->spin_limit = polls;
    return W4_OK;
}

int w4_pass_destroy(w4_pass* p) {
    pass_free(p);
    return W4_OK;
}

}  // extern "C"
