// Acceptance step after the verify pass: the target's K+1 logit rows decide
// how many of the K drafted tokens are kept and which token comes next.
//
// Defined on the explainer page "Speculative Decoding이란?" (section 3, Steps
// 3 and 4; sections 5 and 6): drafted token j is tested against target row j
// -- greedily (it must be the row's argmax) or stochastically (accepted when
// u_j < min(1, p_j(d)/q_j(d))); at the first rejection the next token is the
// row's argmax (greedy) or a draw from the residual max(0, p_j - q_j)
// (stochastic); when all K are accepted it comes from row K.  p and q are the
// softmax of the target and draft logits.
//
// Four launches on the caller's stream, no host synchronisation:
//   accept_stats_kernel   every (row, slice): max, sum of exp(x - max), first
//                         index of the max -- the rows stream once at full
//                         bandwidth, split over ~2K workgroups;
//   accept_decide_kernel  one workgroup: the slices of each row combined in
//                         slice order, then the K sequential tests;
//   accept_sum_kernel     (stochastic only) the sum of the final row's weights
//                         per 1024-element slice;
//   accept_draw_kernel    (stochastic only) the inverse-CDF draw: the slice
//                         holding u * total, then a workgroup scan inside it.
// Every reduction runs in a fixed order, so a call is deterministic.
#include "w4_aux.h"

#include <algorithm>
#include <cmath>

namespace w4 {

namespace {

constexpr int kAccThreads = 256;
constexpr int kDrawSlice = 4 * kAccThreads;  // elements per slice of the final draw

struct RowStat {
    float m;  // max
    float s;  // sum of exp(x - m)
    int i;    // first index of the max
};

// Combine the statistics of two disjoint sets of indices (s == 0: empty).
// Equal maxima keep the smaller index, so any combination order yields the
// first index of the maximum.
__device__ __forceinline__ RowStat combine(RowStat a, RowStat b) {
    if (b.s == 0.0f) return a;
    if (a.s == 0.0f) return b;
    RowStat r;
    r.m = fmaxf(a.m, b.m);
    r.s = a.s * expf(a.m - r.m) + b.s * expf(b.m - r.m);
    r.i = a.m > b.m ? a.i : (b.m > a.m ? b.i : min(a.i, b.i));
    return r;
}

__device__ __forceinline__ RowStat shfl_xor_stat(RowStat v, int mask) {
    RowStat o;
    o.m = __shfl_xor(v.m, mask);
    o.s = __shfl_xor(v.s, mask);
    o.i = __shfl_xor(v.i, mask);
    return o;
}

__device__ RowStat block_combine(RowStat v, RowStat* sh) {
    const int tid = threadIdx.x;
    sh[tid] = v;
    __syncthreads();
    for (int w = kAccThreads / 2; w > 0; w >>= 1) {
        if (tid < w) sh[tid] = combine(sh[tid], sh[tid + w]);
        __syncthreads();
    }
    return sh[0];
}

// Row r < M is target row r, else draft row r - M.  Slice b of a row covers
// [b * per, min(V, (b + 1) * per)), per a multiple of 4; thread t takes the
// quads t, t + 256, ... of the slice (a contiguous 4 KB per pass).
__global__ __launch_bounds__(kAccThreads) void accept_stats_kernel(const float* __restrict__ lt,
                                                                     const float* __restrict__ ld, int M, int V,
                                                                     int per, RowStat* __restrict__ stats) {
    __shared__ RowStat sh[kAccThreads];
    const int b = blockIdx.x, r = blockIdx.y, nb = gridDim.x;
    const float* row = r < M ? lt + (size_t)r * V : ld + (size_t)(r - M) * V;
    const int lo = b * per, hi = min(V, lo + per);
    // first pass: max and its first index
    float m = -INFINITY;
    int mi = 0x7FFFFFFF;
    for (int k = lo + 4 * threadIdx.x; k < hi; k += 4 * kAccThreads) {
        const float4 v = *(const float4*)(row + k);
        if (v.x > m) m = v.x, mi = k;
        if (v.y > m) m = v.y, mi = k + 1;
        if (v.z > m) m = v.z, mi = k + 2;
        if (v.w > m) m = v.w, mi = k + 3;
    }
    // second pass (same bytes, now in L2): sum of exp(x - m) over the thread's elements
    float s = 0.0f;
    if (mi != 0x7FFFFFFF)
        for (int k = lo + 4 * threadIdx.x; k < hi; k += 4 * kAccThreads) {
            const float4 v = *(const float4*)(row + k);
            s += expf(v.x - m) + expf(v.y - m) + expf(v.z - m) + expf(v.w - m);
        }
    const RowStat all = block_combine(RowStat{m, s, mi}, sh);
    if (threadIdx.x == 0) stats[(size_t)r * nb + b] = all;
}

}  // namespace

// Decision state shared by the launches of one call.
struct AcceptState {
    int n;       // drafted tokens accepted
    int row;     // final row to draw from (stochastic), -1 when no draw
    int kind;    // 0: residual max(0, p - q) of target/draft row `row`, 1: p of target row `row`
    int pad;
    float mt, st, md, sd;  // softmax statistics of the final rows
};

namespace {

constexpr int kDecideThreads = 1024;

__global__ __launch_bounds__(kDecideThreads) void accept_decide_kernel(const RowStat* __restrict__ stats, int nb,
                                                                       const float* __restrict__ lt,
                                                                       const float* __restrict__ ld,
                                                                       const int32_t* __restrict__ draft,
                                                                       const float* __restrict__ u, int K, int V,
                                                                       int sampled, int32_t* __restrict__ out,
                                                                       AcceptState* st) {
    __shared__ RowStat rows[2 * kAcceptMaxK + 1];
    __shared__ int pass[kAcceptMaxK];
    const int R = sampled ? 2 * K + 1 : K + 1;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = kDecideThreads / 64;
    // each wave combines whole rows: lanes take slices lane, lane + 64, ...,
    // then a butterfly over the lanes
    for (int r = wave; r < R; r += nw) {
        RowStat a{-INFINITY, 0.0f, 0x7FFFFFFF};
        for (int b = lane; b < nb; b += 64) a = combine(a, stats[(size_t)r * nb + b]);
        for (int mask = 32; mask > 0; mask >>= 1) a = combine(a, shfl_xor_stat(a, mask));
        if (lane == 0) rows[r] = a;
    }
    __syncthreads();
    // the K tests, each independent of the others
    for (int j = threadIdx.x; j < K; j += kDecideThreads) {
        const int d = draft[j];
        const bool valid = d >= 0 && d < V;  // a token outside the vocabulary is rejected
        bool ok;
        if (!sampled) {
            ok = valid && d == rows[j].i;
        } else {
            float alpha = 0.0f;
            if (valid) {
                const RowStat& t = rows[j];
                const RowStat& q = rows[K + 1 + j];
                const float pd = expf(lt[(size_t)j * V + d] - t.m) / t.s;
                const float qd = expf(ld[(size_t)j * V + d] - q.m) / q.s;
                alpha = qd == 0.0f ? 1.0f : fminf(1.0f, pd / qd);
            }
            ok = u[j] < alpha;
        }
        pass[j] = ok;
    }
    __syncthreads();
    if (threadIdx.x != 0) return;
    // accepted in order up to the first rejection
    int n = K, row = K, kind = 1;
    for (int j = 0; j < K; ++j) {
        if (!pass[j]) {
            n = j;
            row = j;
            kind = 0;
            break;
        }
    }
    out[0] = n;
    if (!sampled) {
        out[1] = rows[n].i;
        st->row = -1;
        return;
    }
    out[1] = -1;  // written by the draw
    st->n = n;
    st->row = row;
    st->kind = kind;
    st->mt = rows[row].m;
    st->st = rows[row].s;
    if (kind == 0) {
        st->md = rows[K + 1 + row].m;
        st->sd = rows[K + 1 + row].s;
    }
}

// weight of token k in the final draw
__device__ __forceinline__ float draw_weight(const AcceptState& st, const float* lt, const float* ld, int V, int k) {
    const float p = expf(lt[(size_t)st.row * V + k] - st.mt) / st.st;
    if (st.kind == 1) return p;
    const float q = expf(ld[(size_t)st.row * V + k] - st.md) / st.sd;
    return fmaxf(p - q, 0.0f);
}

__device__ float block_sum(float v, float* sh) {
    const int tid = threadIdx.x;
    sh[tid] = v;
    __syncthreads();
    for (int w = kAccThreads / 2; w > 0; w >>= 1) {
        if (tid < w) sh[tid] += sh[tid + w];
        __syncthreads();
    }
    return sh[0];
}

__global__ __launch_bounds__(kAccThreads) void accept_sum_kernel(const AcceptState* __restrict__ stp,
                                                                   const float* __restrict__ lt,
                                                                   const float* __restrict__ ld, int V,
                                                                   float* __restrict__ part) {
    __shared__ float sh[kAccThreads];
    const AcceptState st = *stp;
    const int lo = blockIdx.x * kDrawSlice + 4 * threadIdx.x;
    float s = 0.0f;
    for (int k = lo; k < min(V, lo + 4); ++k) s += draw_weight(st, lt, ld, V, k);
    s = block_sum(s, sh);
    if (threadIdx.x == 0) part[blockIdx.x] = s;
}

// Inclusive scan of one value per thread (Hillis-Steele in LDS).
__device__ float block_scan(float v, float* sh) {
    const int tid = threadIdx.x;
    sh[tid] = v;
    __syncthreads();
    for (int w = 1; w < kAccThreads; w <<= 1) {
        const float add = tid >= w ? sh[tid - w] : 0.0f;
        __syncthreads();
        sh[tid] += add;
        __syncthreads();
    }
    return sh[tid];
}

// The draw selects, at each of its two levels (slice, then element), the
// lowest thread whose scan interval [exclusive, inclusive) holds the target:
// rounding can make neighbouring intervals overlap, and an LDS atomicMin makes
// the choice unique and the same on every run.  Every thread reads the
// winner into a register after a barrier and branches on that copy, so all
// waves take the same path and meet the same barriers.
__global__ __launch_bounds__(kAccThreads) void accept_draw_kernel(const AcceptState* __restrict__ stp,
                                                                    const float* __restrict__ lt,
                                                                    const float* __restrict__ ld,
                                                                    const float* __restrict__ u, int K, int V,
                                                                    const float* __restrict__ part, int nparts,
                                                                    int32_t* __restrict__ out) {
    __shared__ float sh[kAccThreads];
    __shared__ int win;
    __shared__ int pick_slice, pick;
    __shared__ float base;
    const AcceptState st = *stp;
    const int tid = threadIdx.x;
    // slice sums: thread t holds slices [t*c, (t+1)*c) in order
    const int c = (nparts + kAccThreads - 1) / kAccThreads;
    float mine = 0.0f;
    for (int b = tid * c; b < min(nparts, (tid + 1) * c); ++b) mine += part[b];
    const float incl = block_scan(mine, sh);
    const float total = sh[kAccThreads - 1];
    const float target = u[K] * total;
    if (tid == 0) win = kAccThreads;
    __syncthreads();
    const float excl = incl - mine;
    if (mine > 0.0f && excl <= target && target < incl) atomicMin(&win, tid);
    __syncthreads();
    const int w1 = win;  // uniform
    if (w1 < kAccThreads) {
        // the winning thread walks its slices to the one that crosses the target
        if (tid == w1) {
            float acc = excl;
            int b = tid * c;
            for (; b < min(nparts, (tid + 1) * c) - 1; ++b) {
                if (acc + part[b] > target) break;
                acc += part[b];
            }
            pick_slice = b;
            base = acc;
        }
    } else if (tid == 0) {
        // rounding put the target at (or past) the total: the last slice with weight
        int b = nparts - 1;
        while (b > 0 && part[b] <= 0.0f) --b;
        float acc = 0.0f;
        for (int i = 0; i < b; ++i) acc += part[i];
        pick_slice = b;
        base = acc;
    }
    __syncthreads();
    const int ps = pick_slice;
    const float b0 = base;
    // scan inside the slice: thread t holds its 4 consecutive elements
    const int lo = ps * kDrawSlice + 4 * tid;
    float w4v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    float s = 0.0f;
    for (int k = 0; k < 4; ++k)
        if (lo + k < V) {
            w4v[k] = draw_weight(st, lt, ld, V, lo + k);
            s += w4v[k];
        }
    const float in2 = block_scan(s, sh) + b0;
    if (tid == 0) win = kAccThreads;
    __syncthreads();
    const float ex2 = in2 - s;
    if (s > 0.0f && ex2 <= target && target < in2) atomicMin(&win, tid);
    __syncthreads();
    const int w2 = win;  // uniform
    if (w2 < kAccThreads) {
        if (tid == w2) {
            float acc = ex2;
            int k = 0;
            for (; k < 3; ++k) {
                if (w4v[k] > 0.0f && acc + w4v[k] > target) break;
                acc += w4v[k];
            }
            while (k > 0 && w4v[k] <= 0.0f) --k;
            pick = lo + k;
        }
    } else if (tid == 0) {
        // rounding: the last element of the slice with weight
        int k = min(V, (ps + 1) * kDrawSlice) - 1;
        while (k > ps * kDrawSlice && draw_weight(st, lt, ld, V, k) <= 0.0f) --k;
        pick = k;
    }
    __syncthreads();
    if (tid == 0) out[1] = pick;
}

int stats_slices(int rows, int V) {
    // ~2048 workgroups in all, at least 4 KB per slice, at most 256 slices
    const int want = std::max(1, 2048 / std::max(1, rows));
    const int most = std::max(1, (V + 1023) / 1024);
    return std::min(std::min(want, most), 256);
}

template <typename... Args>
hipError_t launch(void (*kernel)(Args...), dim3 grid, dim3 block, hipStream_t stream, Args... args) {
    void* argv[] = {(void*)&args...};
    return hipLaunchKernel((const void*)kernel, grid, block, argv, 0, stream);
}

}  // namespace

size_t accept_workspace_bytes(int K, int V) {
    const int rows = 2 * K + 1;
    const size_t stats = (size_t)rows * stats_slices(rows, V) * sizeof(RowStat);
    const size_t parts = (size_t)((V + kDrawSlice - 1) / kDrawSlice) * sizeof(float);
    return 256 + ((stats + 255) / 256) * 256 + parts;
}

hipError_t launch_accept(const float* lt, const float* ld, const int32_t* draft, const float* u, int K, int V,
                         int sampled, int32_t* out, void* ws, hipStream_t stream) {
    const int M = K + 1;
    const int rows = sampled ? 2 * K + 1 : M;
    const int nb = stats_slices(2 * K + 1, V);
    int per = (V + nb - 1) / nb;
    per = (per + 3) & ~3;
    char* base = (char*)ws;
    AcceptState* st = (AcceptState*)base;
    RowStat* stats = (RowStat*)(base + 256);
    const size_t stats_bytes = (((size_t)(2 * K + 1) * nb * sizeof(RowStat) + 255) / 256) * 256;
    float* part = (float*)(base + 256 + stats_bytes);
    hipError_t e = launch(accept_stats_kernel, dim3(nb, rows), dim3(kAccThreads), stream, lt, ld, M, V, per, stats);
    if (e != hipSuccess) return e;
    e = launch(accept_decide_kernel, dim3(1), dim3(kDecideThreads), stream, (const RowStat*)stats, nb, lt, ld, draft,
               u, K, V, sampled, out, st);
    if (e != hipSuccess || !sampled) return e;
    const int nparts = (V + kDrawSlice - 1) / kDrawSlice;
    e = launch(accept_sum_kernel, dim3(nparts), dim3(kAccThreads), stream, (const AcceptState*)st, lt, ld, V, part);
    if (e != hipSuccess) return e;
    return launch(accept_draw_kernel, dim3(1), dim3(kAccThreads), stream, (const AcceptState*)st, lt, ld, u, K, V,
                  (const float*)part, nparts, out);
}

}  // namespace w4
