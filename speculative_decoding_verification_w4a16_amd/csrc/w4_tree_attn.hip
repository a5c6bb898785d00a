// Tree-draft verify attention: M draft tokens (a flattened tree) attend to a
// KV prefix of L positions and to the draft tokens set in their ancestor
// masks, with grouped query heads (Llama-3-70B: 64 query heads over 8
// key/value heads, head dim 128).
//
// The pages describe the step only in words (the review page's "Compatibility
// Problem": tree verification holds several candidates and verifies them in
// parallel; the explainer page "Speculative Decoding이란?", sections 8 and
// 10.1: a tree of candidates checked by the target at once, Medusa's
// tree-based attention).  Reading: token i sees every prefix position and
// draft token j iff bit j of mask[i] is set; softmax(q.k * scale) over what it
// sees; query head h reads key/value head h / (Hq / Hkv).
//
// Layout of the work.  The rows of key/value head g are the M x G (token,
// query head) pairs that read it, row = token * G + head-in-group; a
// workgroup of 4 waves takes 64 rows (16 per wave) over a contiguous run of
// 64-key chunks of the key sequence (the L prefix positions, then the M draft
// tokens).  Per chunk and wave, both products run on bf16 MFMA (16x16x32):
//
//   scores, transposed: S^T[key][row] = K[key][:] . Q[row][:] -- the A
//   operand is 8 consecutive head-dim values of one key and the B operand 8
//   of one row, both contiguous 16-byte loads; the result gives each lane one
//   row (lane % 16) and four keys, so the online softmax of a row reduces over
//   the four lanes that share it (two shuffles);
//   output, transposed: O^T[d][row] += V^T[d][key] . P^T[key][row] -- the B
//   operand is the lane's own probabilities in bf16 (an MFMA sums over k in
//   any order as long as A and B agree, so the lane's keys need no
//   rearranging), the A operand 8 keys of one head-dim column, read from an
//   LDS copy of the chunk's V stored column-major (d, key): pairs of keys are
//   packed into dwords with v_perm_b32 on the way in.
//
// Each workgroup writes its unnormalised output with the running max and sum
// of each row; tree_attn_combine_kernel merges the key splits (log-sum-exp).
#include "w4_aux.h"

#include <algorithm>
#include <cmath>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

namespace w4 {

namespace {

constexpr int kHd = kTreeHeadDim;  // 128
constexpr int kChunk = 64;         // keys per chunk
constexpr int kRowsWg = 64;        // query rows per workgroup (16 per wave)
constexpr int kVtPitch = kChunk * 2 + 8;  // bytes per head-dim column of the V copy (padded against bank conflicts)
constexpr int kVtBytes = kHd * kVtPitch;  // one chunk's V copy

struct TreeArgs {
    const uint16_t* q;   // [M][Hq][128]
    const uint16_t* kc;  // [L][Hkv][128]
    const uint16_t* vc;
    const uint16_t* kd;  // [M][Hkv][128]
    const uint16_t* vd;
    const uint64_t* masks;  // [M]
    float* opart;        // [S][Hkv][R][128]
    float* mpart;        // [S][Hkv][R]
    float* lpart;        // [S][Hkv][R]
    float* out;          // [M][Hq][128]
    int M, L, Hq, Hkv, G, R, T;
    int nchunks, cps, nsplit;
    float scale;
};

// 16 bytes (8 head-dim values starting at d) of key/value position `key` of
// head g: prefix positions first, then the draft tokens.
__device__ __forceinline__ u32x4 kv_load(const uint16_t* cache, const uint16_t* draft, const TreeArgs& a, int key,
                                         int g, int d) {
    const uint16_t* p = key < a.L ? cache + ((size_t)key * a.Hkv + g) * kHd + d
                                  : draft + ((size_t)(key - a.L) * a.Hkv + g) * kHd + d;
    return *(const u32x4*)p;
}

__global__ __launch_bounds__(256) void tree_attn_partial_kernel(TreeArgs a) {
    __shared__ __align__(16) char vt[2 * kVtBytes];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int o = lane >> 4, t = lane & 15;
    const int split = blockIdx.x, rt = blockIdx.y, g = blockIdx.z;
    const int row = rt * kRowsWg + 16 * wave + t;  // this lane's row
    const bool row_ok = row < a.R;
    const int tok = row_ok ? row / a.G : 0;
    const int head = g * a.G + (row_ok ? row % a.G : 0);
    const uint64_t mask = row_ok ? a.masks[tok] : 0ull;

    // B operands of the scores: the row's 128 head-dim values, 8 per lane per k-block
    bf16x8 qb[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        const u32x4 v = *(const u32x4*)(a.q + ((size_t)tok * a.Hq + head) * kHd + 32 * kb + 8 * o);
        qb[kb] = __builtin_bit_cast(bf16x8, row_ok ? v : u32x4{0, 0, 0, 0});
    }
    f32x4 oacc[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oacc[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -INFINITY, l_run = 0.0f;

    // Chunk loads: the thread's two V items (key pairs of one head-dim octet)
    // and the lane's K operands of the four score tiles.  Chunk c+1's V is
    // loaded as soon as chunk c's is in LDS, its K once chunk c's scores are
    // issued (into the same registers), so both arrive while chunk c
    // computes; the V copy alternates between two LDS buffers, so one
    // barrier per chunk orders both its writes and the buffer's reuse.
    struct ChunkRegs {
        u32x4 va[2], vb[2];
        u32x4 k[4][4];
    };
    const int c0 = split * a.cps, c1 = min(a.nchunks, c0 + a.cps);
    auto load_v = [&](ChunkRegs& r, int c) {
        const int key0 = c * kChunk;
#pragma unroll
        for (int rep = 0; rep < 2; ++rep) {
            const int item = threadIdx.x + 256 * rep;
            const int p = item & 31, qd = item >> 5;
            const int k0 = key0 + 2 * p;
            // past the end: a valid address, the value replaced by zero
            const u32x4 x0 = kv_load(a.vc, a.vd, a, min(k0, a.T - 1), g, 8 * qd);
            const u32x4 x1 = kv_load(a.vc, a.vd, a, min(k0 + 1, a.T - 1), g, 8 * qd);
            r.va[rep] = k0 < a.T ? x0 : u32x4{0, 0, 0, 0};
            r.vb[rep] = k0 + 1 < a.T ? x1 : u32x4{0, 0, 0, 0};
        }
    };
    auto load_k = [&](ChunkRegs& r, int c) {
        const int key0 = c * kChunk;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            const int key = min(key0 + 16 * kt + t, a.T - 1);  // masked below when past the end
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) r.k[kt][kb] = kv_load(a.kc, a.kd, a, key, g, 32 * kb + 8 * o);
        }
    };
    auto step = [&](ChunkRegs& cur, ChunkRegs& nxt, int c) {
        const int key0 = c * kChunk;
        char* buf = vt + (c & 1) * kVtBytes;
        // V of the chunk into LDS, column-major: dword (d, key pair p) holds keys 2p, 2p+1
#pragma unroll
        for (int rep = 0; rep < 2; ++rep) {
            const int item = threadIdx.x + 256 * rep;
            const int p = item & 31, qd = item >> 5;
#pragma unroll
            for (int w2 = 0; w2 < 4; ++w2) {
                const uint32_t lo = __builtin_amdgcn_perm(cur.vb[rep][w2], cur.va[rep][w2], 0x05040100u);
                const uint32_t hi = __builtin_amdgcn_perm(cur.vb[rep][w2], cur.va[rep][w2], 0x07060302u);
                *(uint32_t*)(buf + (8 * qd + 2 * w2) * kVtPitch + 4 * p) = lo;      // d = 8qd + 2w2
                *(uint32_t*)(buf + (8 * qd + 2 * w2 + 1) * kVtPitch + 4 * p) = hi;  // d = 8qd + 2w2 + 1
            }
        }
        if (c + 1 < c1) load_v(nxt, c + 1);
        // scores of the chunk's four 16-key tiles
        f32x4 s[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.k[kt][kb]), qb[kb], acc,
                                                              0, 0, 0);
            s[kt] = acc;
        }
        // the next chunk's K operands reuse the registers of this chunk's
        if (c + 1 < c1) load_k(nxt, c + 1);
        // scale and mask: lane (o, t) holds keys key0 + 16kt + 4o + r of row t
        float cm = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = key0 + 16 * kt + 4 * o + r;
                bool vis = key < a.T;
                if (key >= a.L) vis = vis && ((mask >> (unsigned)(key - a.L)) & 1ull);
                const float v = vis ? s[kt][r] * a.scale : -INFINITY;
                s[kt][r] = v;
                cm = fmaxf(cm, v);
            }
        cm = fmaxf(cm, __shfl_xor(cm, 16));
        cm = fmaxf(cm, __shfl_xor(cm, 32));
        const float m_new = fmaxf(m_run, cm);
        const bool none = m_new == -INFINITY;  // nothing visible to this row yet
        const float alpha = none ? 1.0f : expf(m_run - m_new);
        float ls = 0.0f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = none ? 0.0f : expf(s[kt][r] - m_new);
                s[kt][r] = p;
                ls += p;
            }
        ls += __shfl_xor(ls, 16);
        ls += __shfl_xor(ls, 32);
        l_run = l_run * alpha + ls;
        m_run = m_new;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) oacc[dt] *= alpha;
        __syncthreads();  // the V copy of chunk c is complete (and chunk c-1's copy is no longer read)
        // O^T += V^T P^T over the chunk's two 32-key halves
#pragma unroll
        for (int kp = 0; kp < 2; ++kp) {
            bf16x8 pb;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                pb[r] = (__bf16)s[2 * kp][r];
                pb[4 + r] = (__bf16)s[2 * kp + 1][r];
            }
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                const char* col = buf + (16 * dt + t) * kVtPitch;
                const uint2 lo = *(const uint2*)(col + 2 * (32 * kp + 4 * o));
                const uint2 hi = *(const uint2*)(col + 2 * (32 * kp + 16 + 4 * o));
                const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
                oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, oacc[dt], 0, 0, 0);
            }
        }
    };
    ChunkRegs ra, rb;
    if (c0 < c1) {
        load_v(ra, c0);
        load_k(ra, c0);
    }
    for (int c = c0; c < c1; c += 2) {
        step(ra, rb, c);
        if (c + 1 < c1) step(rb, ra, c + 1);
    }

    if (row_ok) {
        const size_t base = ((size_t)split * a.Hkv + g) * a.R + row;
        float* op = a.opart + base * kHd;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) op[16 * dt + 4 * o + r] = oacc[dt][r];
        if (o == 0) {
            a.mpart[base] = m_run;
            a.lpart[base] = l_run;
        }
    }
}

// out[tok][head][d] = sum_s e^(m_s - m) O_s / sum_s e^(m_s - m) l_s, over the key splits
__global__ __launch_bounds__(256) void tree_attn_combine_kernel(TreeArgs a) {
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t total = (size_t)a.Hkv * a.R * kHd;
    if (idx >= total) return;
    const int d = (int)(idx % kHd);
    const size_t gr = idx / kHd;  // g * R + row
    const int row = (int)(gr % a.R), g = (int)(gr / a.R);
    const size_t plane = (size_t)a.Hkv * a.R;
    // the splits' loads are independent: unrolled so that many are in flight
    float m = -INFINITY;
#pragma unroll 8
    for (int s = 0; s < a.nsplit; ++s) m = fmaxf(m, a.mpart[s * plane + gr]);
    float num = 0.0f, den = 0.0f;
    if (m != -INFINITY) {
#pragma unroll 8
        for (int s = 0; s < a.nsplit; ++s) {
            const float w = expf(a.mpart[s * plane + gr] - m);
            num += w * a.opart[(s * plane + gr) * kHd + d];
            den += w * a.lpart[s * plane + gr];
        }
    }
    const int tok = row / a.G, head = g * a.G + row % a.G;
    a.out[((size_t)tok * a.Hq + head) * kHd + d] = den > 0.0f ? num / den : 0.0f;
}

template <typename... Args>
hipError_t launch(void (*kernel)(Args...), dim3 grid, dim3 block, hipStream_t stream, Args... args) {
    void* argv[] = {(void*)&args...};
    return hipLaunchKernel((const void*)kernel, grid, block, argv, 0, stream);
}

}  // namespace

int tree_attn_plan(int M, int L, int Hq, int Hkv, int* nsplit_out, size_t* ws_bytes) {
    const int G = Hq / Hkv, R = M * G, T = L + M;
    const int nchunks = (T + kChunk - 1) / kChunk;
    const int nrt = (R + kRowsWg - 1) / kRowsWg;
    // ~256 workgroups (the chunks of a split are pipelined, so long splits
    // cost little; every split adds combine work), at most what the
    // workspace holds
    int nsplit = std::max(1, std::min(nchunks, (256 + nrt * Hkv - 1) / (nrt * Hkv)));
    const auto bytes = [&](int s) { return (size_t)s * Hkv * R * (kHd + 2) * sizeof(float); };
    while (nsplit > 1 && bytes(nsplit) > kTreeWorkspaceBytes) --nsplit;
    const int cps = (nchunks + nsplit - 1) / nsplit;
    nsplit = (nchunks + cps - 1) / cps;
    if (nsplit_out) *nsplit_out = nsplit;
    if (ws_bytes) *ws_bytes = bytes(nsplit);
    return bytes(nsplit) <= kTreeWorkspaceBytes ? 0 : -1;
}

hipError_t launch_tree_attn(const uint16_t* q, const uint16_t* kc, const uint16_t* vc, const uint16_t* kd,
                            const uint16_t* vd, const uint64_t* masks, int M, int L, int Hq, int Hkv, float scale,
                            float* out, void* ws, hipStream_t stream) {
    TreeArgs a;
    a.q = q;
    a.kc = kc;
    a.vc = vc;
    a.kd = kd;
    a.vd = vd;
    a.masks = masks;
    a.M = M;
    a.L = L;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = Hq / Hkv;
    a.R = M * a.G;
    a.T = L + M;
    a.nchunks = (a.T + kChunk - 1) / kChunk;
    tree_attn_plan(M, L, Hq, Hkv, &a.nsplit, nullptr);
    a.cps = (a.nchunks + a.nsplit - 1) / a.nsplit;
    a.scale = scale;
    const size_t plane = (size_t)a.nsplit * Hkv * a.R;
    a.opart = (float*)ws;
    a.mpart = a.opart + plane * kHd;
    a.lpart = a.mpart + plane;
    a.out = out;
    const int nrt = (a.R + kRowsWg - 1) / kRowsWg;
    hipError_t e = launch(tree_attn_partial_kernel, dim3(a.nsplit, nrt, Hkv), dim3(256), stream, a);
    if (e != hipSuccess) return e;
    const size_t total = (size_t)Hkv * a.R * kHd;
    return launch(tree_attn_combine_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), stream, a);
}

}  // namespace w4
