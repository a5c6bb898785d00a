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
// workgroup of W waves takes 16W rows (16 per wave; W = 4 when the rows of a
// head fit one wave, else 8, which halves the chunk copies per row) over a
// contiguous run of
// 64-key chunks of the key sequence (the L prefix positions, then the M draft
// tokens).  The workgroup copies each chunk's keys and values into LDS once
// (registers -> LDS, the next chunk's loads in flight meanwhile; two
// buffers, one barrier per chunk), and every wave reads its MFMA operands
// there.  Per chunk and wave, both products run on bf16 MFMA (16x16x32):
//
//   scores, transposed: S^T[key][row] = K[key][:] . Q[row][:] -- the A
//   operand is 8 consecutive head-dim values of one key (a 16-byte LDS read,
//   key rows padded to 272 bytes so sixteen keys fall in distinct banks), the
//   B operand 8 of the wave's row, kept in registers; the result gives each
//   lane one row (lane % 16) and four keys, so the online softmax of a row
//   reduces over the four lanes that share it (two shuffles);
//   output, transposed: O^T[d][row] += V^T[d][key] . P^T[key][row] -- the B
//   operand is the lane's own probabilities in bf16 (an MFMA sums over k in
//   any order as long as A and B agree, so the lane's keys need no
//   rearranging), the A operand 8 keys of one head-dim column, read from the
//   LDS copy of V stored column-major (d, key pair): pairs of keys are packed
//   into dwords with v_perm_b32 on the way in, and the pair index is XORed
//   with a multiple of 4 that depends on d so that the writes of sixteen
//   columns spread over the banks.
//
// The softmax runs in base 2: scores are scaled by scale * log2(e) and
// exponentiated with the hardware exp2.  With one key split a workgroup
// writes its normalised rows; otherwise each writes its unnormalised output
// with the running max and sum of every row, and tree_attn_combine_kernel
// merges the splits (log-sum-exp), one workgroup per row.
#include "w4_aux.h"

#include <algorithm>
#include <cmath>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

namespace w4 {

namespace {

constexpr int kHd = kTreeHeadDim;              // 128
constexpr int kChunk = 64;                     // keys per chunk
constexpr int kKPitch = kHd * 2 + 16;          // bytes per key row of the K copy
constexpr int kKBytes = kChunk * kKPitch;      // one chunk's K copy
constexpr int kVtPitch = kChunk * 2 + 8;       // bytes per head-dim column of the V copy
constexpr int kVtBytes = kHd * kVtPitch;       // one chunk's V copy
constexpr int kBufBytes = kKBytes + kVtBytes;  // one LDS buffer (K then V)
constexpr float kLog2e = 1.4426950408889634f;

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
    int M, L, Hq, Hkv, G, R, T, nrt;
    int nchunks, nsplit, cng;  // cng: thread groups per row in the merge
    float c;  // scale * log2(e)
};

// 16 bytes (8 head-dim values starting at d) of key/value position `key` of
// head g: prefix positions first, then the draft tokens.
__device__ __forceinline__ u32x4 kv_load(const uint16_t* cache, const uint16_t* draft, const TreeArgs& a, int key,
                                         int g, int d) {
    const uint16_t* p = key < a.L ? cache + ((size_t)key * a.Hkv + g) * kHd + d
                                  : draft + ((size_t)(key - a.L) * a.Hkv + g) * kHd + d;
    return *(const u32x4*)p;
}

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

template <int W>
__global__ __launch_bounds__(64 * W) void tree_attn_kernel(TreeArgs a) {
    constexpr int kRowsWg = 16 * W;  // query rows per workgroup
    __shared__ __align__(16) char smem[2 * kBufBytes];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int o = lane >> 4, t = lane & 15;
    const int split = blockIdx.x, rt = blockIdx.y, g = blockIdx.z;
    const int row = rt * kRowsWg + 16 * wave + t;  // this lane's row
    const bool active = rt * kRowsWg + 16 * wave < a.R;  // the wave has a row (wave-uniform)
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

    // Chunk loads: thread (lt, lq) = (tid / 16, tid % 16) fetches head-dim octet
    // lq of keys lt + 4W r (r < 16/W) and of the value key pairs lt + 4W i
    // (i < 8/W).
    static_assert(W == 4 || W == 8, "4 or 8 waves per workgroup");
    constexpr int KI = 16 / W, VI = 8 / W, TS = 4 * W;  // TS: thread rows (lt) per workgroup
    const int lt = tid >> 4, lq = tid & 15;
    struct ChunkRegs {
        u32x4 k[KI], v[2 * VI];  // v[2i], v[2i+1]: keys 2(lt + TS i) and 2(lt + TS i) + 1
    };
    // a chunk inside the prefix: one wave-uniform base and fixed lane offsets
    const uint32_t pos_bytes = (uint32_t)a.Hkv * kHd * 2;  // between consecutive positions
    const uint32_t lane_k = lt * pos_bytes + g * kHd * 2 + 16 * lq;
    const uint32_t lane_v = 2 * lt * pos_bytes + g * kHd * 2 + 16 * lq;
    auto load = [&](ChunkRegs& cr, int c) {
        const int key0 = c * kChunk;
        if (key0 + kChunk <= a.L) {
            const char* kb = (const char*)a.kc + (size_t)key0 * pos_bytes;
            const char* vb = (const char*)a.vc + (size_t)key0 * pos_bytes;
#pragma unroll
            for (int r = 0; r < KI; ++r) cr.k[r] = *(const u32x4*)(kb + (lane_k + TS * r * pos_bytes));
#pragma unroll
            for (int r = 0; r < 2 * VI; ++r)
                cr.v[r] = *(const u32x4*)(vb + (lane_v + (2 * TS * (r >> 1) + (r & 1)) * pos_bytes));
        } else {
#pragma unroll
            for (int r = 0; r < KI; ++r) cr.k[r] = kv_load(a.kc, a.kd, a, min(key0 + lt + TS * r, a.T - 1), g, 8 * lq);
#pragma unroll
            for (int r = 0; r < 2 * VI; ++r)
                cr.v[r] = kv_load(a.vc, a.vd, a, min(key0 + 2 * (lt + TS * (r >> 1)) + (r & 1), a.T - 1), g, 8 * lq);
        }
    };
    // ... into LDS buffer b.  Keys past the end keep a valid (clamped) K row,
    // masked later, and a zero V row.
    const int vsw = 4 * ((lq >> 2) & 3);  // pair swizzle of the thread's columns 8lq..8lq+7
    auto store = [&](ChunkRegs& cr, int b, int c) {
        char* kbuf = smem + b * kBufBytes;
        char* vbuf = kbuf + kKBytes;
#pragma unroll
        for (int r = 0; r < KI; ++r) *(u32x4*)(kbuf + (lt + TS * r) * kKPitch + 16 * lq) = cr.k[r];
        if (c * kChunk + kChunk > a.T) {
#pragma unroll
            for (int r = 0; r < 2 * VI; ++r)
                if (c * kChunk + 2 * (lt + TS * (r >> 1)) + (r & 1) >= a.T) cr.v[r] = u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < VI; ++i) {
            const int p = (lt + TS * i) ^ vsw;
#pragma unroll
            for (int w2 = 0; w2 < 4; ++w2) {
                const uint32_t lo = __builtin_amdgcn_perm(cr.v[2 * i + 1][w2], cr.v[2 * i][w2], 0x05040100u);
                const uint32_t hi = __builtin_amdgcn_perm(cr.v[2 * i + 1][w2], cr.v[2 * i][w2], 0x07060302u);
                *(uint32_t*)(vbuf + (8 * lq + 2 * w2) * kVtPitch + 4 * p) = lo;      // d = 8lq + 2w2
                *(uint32_t*)(vbuf + (8 * lq + 2 * w2 + 1) * kVtPitch + 4 * p) = hi;  // d = 8lq + 2w2 + 1
            }
        }
    };

    // LDS read offsets of the lane: K rows t (+16kt), octet o (+4kb); V^T
    // column t (+16dt), key pairs 2o, 2o+1 (lo) and 8+2o, 9+2o (hi) of each
    // 16-pair half, swizzled by s = 4((dt >> 1) & 3)
    const int koff = t * kKPitch + 16 * o;
    int vlo[4], vhi[4];
#pragma unroll
    for (int si = 0; si < 4; ++si) {
        vlo[si] = kKBytes + t * kVtPitch + 4 * ((2 * o) ^ (4 * si));
        vhi[si] = kKBytes + t * kVtPitch + 4 * ((2 * o + 8) ^ (4 * si));
    }

    // the four lanes of a row: lane ^ 16, lane ^ 32 (byte addresses for ds_bpermute)
    const int x16 = (lane ^ 16) << 2, x32 = (lane ^ 32) << 2;
    auto row_max = [&](float v) {
        v = fmaxf(v, __int_as_float(__builtin_amdgcn_ds_bpermute(x16, __float_as_int(v))));
        return fmaxf(v, __int_as_float(__builtin_amdgcn_ds_bpermute(x32, __float_as_int(v))));
    };
    auto compute = [&](int b, int c) {
        const char* buf = smem + b * kBufBytes;
        const int key0 = c * kChunk;
        // scores of the chunk's four 16-key tiles
        f32x4 s[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const bf16x8 kv = __builtin_bit_cast(bf16x8, *(const u32x4*)(buf + koff + 16 * kt * kKPitch + 64 * kb));
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qb[kb], acc, 0, 0, 0);
            }
            s[kt] = acc;
        }
        // online softmax in base 2: lane (o, t) holds keys key0 + 16kt + 4o + r of row t
        float m_new, alpha;
        if (key0 + kChunk <= a.L) {
            // every key is a prefix position: all visible, all finite
            float cm = s[0][0];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) cm = fmaxf(cm, s[kt][r]);
            m_new = fmaxf(m_run, row_max(cm) * a.c);
            alpha = exp2_hw(m_run - m_new);
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) s[kt][r] = exp2_hw(fmaf(s[kt][r], a.c, -m_new));
        } else {
            float cm = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int key = key0 + 16 * kt + 4 * o + r;
                    bool vis = key < a.T;
                    if (key >= a.L) vis = vis && ((mask >> (unsigned)(key - a.L)) & 1ull);
                    const float v = vis ? s[kt][r] * a.c : -INFINITY;
                    s[kt][r] = v;
                    cm = fmaxf(cm, v);
                }
            m_new = fmaxf(m_run, row_max(cm));
            const bool none = m_new == -INFINITY;  // nothing visible to this row yet
            alpha = none ? 1.0f : exp2_hw(m_run - m_new);
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) s[kt][r] = none ? 0.0f : exp2_hw(s[kt][r] - m_new);
        }
        // the lane's share of the row sum (the four shares are added at the end)
        float ls = 0.0f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) ls += s[kt][r];
        l_run = l_run * alpha + ls;
        m_run = m_new;
        if (__any(alpha != 1.0f)) {  // the running max moved for some row of the wave
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) oacc[dt] *= alpha;
        }
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
                const int si = (dt >> 1) & 3;
                const uint2 lo = *(const uint2*)(buf + vlo[si] + 16 * dt * kVtPitch + 64 * kp);
                const uint2 hi = *(const uint2*)(buf + vhi[si] + 16 * dt * kVtPitch + 64 * kp);
                const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
                oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, oacc[dt], 0, 0, 0);
            }
        }
    };

    // chunks [c0, c1) of the key sequence, spread evenly over the splits
    const int c0 = (int)((long long)split * a.nchunks / a.nsplit);
    const int c1 = (int)((long long)(split + 1) * a.nchunks / a.nsplit);
    // the next chunk's loads fly while this one is stored and computed
    ChunkRegs cr;
    load(cr, c0);
    for (int c = c0; c < c1; ++c) {
        const int b = (c - c0) & 1;
        store(cr, b, c);
        if (c + 1 < c1) load(cr, c + 1);
        __syncthreads();  // chunk c is in buffer b; buffer b's previous chunk is no longer read
        if (active) compute(b, c);
    }

    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    if (a.nsplit == 1) {
        if (row_ok) {
            const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
            float* op = a.out + ((size_t)tok * a.Hq + head) * kHd + 4 * o;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) *(f32x4*)(op + 16 * dt) = oacc[dt] * inv;
        }
        return;
    }
    const size_t plane = (size_t)a.Hkv * a.R;
    if (row_ok) {
        const size_t base = (size_t)split * plane + (size_t)g * a.R + row;
        float* op = a.opart + base * kHd + 4 * o;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) *(f32x4*)(op + 16 * dt) = oacc[dt];
        if (o == 0) {
            a.mpart[base] = m_run;
            a.lpart[base] = l_run;
        }
    }
}

// out[tok][head][:] = sum_s 2^(m_s - m) O_s / sum_s 2^(m_s - m) l_s over the
// key splits, m = max_s m_s.  A group of 32 threads holds one row (a float4
// each); a row has ng = 1, 2, 4 or 8 groups (the fewest that leave at most
// eight splits per group), each taking every ng-th split with all its loads
// issued at once; the first group of the row merges the ng results.  A
// workgroup holds 8 / ng rows.
static_assert(kTreeMaxSplits <= 64, "at most eight splits per thread group");
__global__ __launch_bounds__(256) void tree_attn_combine_kernel(TreeArgs a) {
    const int ng = a.cng;
    const int grp = threadIdx.x >> 5, d4 = threadIdx.x & 31;
    const int sub = grp & (ng - 1);
    const int gr = blockIdx.x * (8 / ng) + grp / ng;  // g * R + row
    const bool ok = gr < a.Hkv * a.R;
    const size_t plane = (size_t)a.Hkv * a.R;
    float ms[8], ls[8];
    f32x4 os[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int sp = sub + ng * j;
        ms[j] = -INFINITY;
        ls[j] = 0.0f;
        os[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if (ok && sp < a.nsplit) {
            const size_t idx = sp * plane + gr;
            ms[j] = a.mpart[idx];
            ls[j] = a.lpart[idx];
            os[j] = *(const f32x4*)(a.opart + idx * kHd + 4 * d4);
        }
    }
    float m = ms[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) m = fmaxf(m, ms[j]);
    float den = 0.0f;
    f32x4 num = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if (m != -INFINITY) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float w = exp2_hw(ms[j] - m);
            num += os[j] * w;
            den += ls[j] * w;
        }
    }
    if (ng > 1) {
        __shared__ float gm[8], gd[8];
        __shared__ f32x4 gn[8][32];
        if (d4 == 0) {
            gm[grp] = m;
            gd[grp] = den;
        }
        gn[grp][d4] = num;
        __syncthreads();
        if (sub != 0) return;
        float mx = -INFINITY;
        for (int k = 0; k < ng; ++k) mx = fmaxf(mx, gm[grp + k]);
        num = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        den = 0.0f;
        if (mx != -INFINITY) {
            for (int k = 0; k < ng; ++k) {
                const float f = exp2_hw(gm[grp + k] - mx);
                num += gn[grp + k][d4] * f;
                den += gd[grp + k] * f;
            }
        }
    }
    if (!ok) return;
    const int g = gr / a.R, row = gr % a.R;
    const int tok = row / a.G, head = g * a.G + row % a.G;
    *(f32x4*)(a.out + ((size_t)tok * a.Hq + head) * kHd + 4 * d4) =
        den > 0.0f ? num * (1.0f / den) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
}

template <typename... Args>
hipError_t launch(void (*kernel)(Args...), dim3 grid, dim3 block, hipStream_t stream, Args... args) {
    void* argv[] = {(void*)&args...};
    return hipLaunchKernel((const void*)kernel, grid, block, argv, 0, stream);
}

size_t partial_bytes(int nsplit, int Hkv, int R) { return (size_t)nsplit * Hkv * R * (kHd + 2) * sizeof(float); }

// Waves per workgroup for R rows per head: 4 (64 rows) when the rows fit one
// wave, else 8 (128 rows).
int tree_waves(int R) { return R > 16 ? 8 : 4; }

}  // namespace

int tree_attn_plan(int M, int L, int Hq, int Hkv, int* nsplit_out, size_t* ws_bytes) {
    const int G = Hq / Hkv, R = M * G, T = L + M;
    const int nchunks = (T + kChunk - 1) / kChunk;
    const int W = tree_waves(R), rows_wg = 16 * W;
    const int nrt = (R + rows_wg - 1) / rows_wg;
    const int tiles = nrt * Hkv;
    // workgroups at once: two of four waves per CU (LDS), one of eight
    // (registers).  Chunks per split: at least two (a workgroup overlaps a
    // chunk's loads with the previous chunk's work), else the fewest that
    // keep to one such round; then at most kTreeMaxSplits splits and what
    // the workspace holds
    const long long slots = W == 4 ? 512 : 256;
    const int cps = std::max(2, (int)(((long long)nchunks * tiles + slots - 1) / slots));
    int nsplit = std::max(1, std::min(kTreeMaxSplits, (nchunks + cps - 1) / cps));
    while (nsplit > 1 && partial_bytes(nsplit, Hkv, R) > kTreeWorkspaceBytes) --nsplit;
    if (nsplit_out) *nsplit_out = nsplit;
    if (ws_bytes) *ws_bytes = nsplit > 1 ? partial_bytes(nsplit, Hkv, R) : 0;
    return 0;
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
    const int W = tree_waves(a.R);
    a.nrt = (a.R + 16 * W - 1) / (16 * W);
    a.nchunks = (a.T + kChunk - 1) / kChunk;
    if (tree_attn_plan(M, L, Hq, Hkv, &a.nsplit, nullptr) != 0) return hipErrorInvalidValue;
    a.c = scale * kLog2e;
    const size_t plane = (size_t)a.nsplit * Hkv * a.R;
    a.opart = (float*)ws;
    a.mpart = a.opart + plane * kHd;
    a.lpart = a.mpart + plane;
    a.out = out;
    hipError_t e = W == 4 ? launch(tree_attn_kernel<4>, dim3(a.nsplit, a.nrt, Hkv), dim3(256), stream, a)
                          : launch(tree_attn_kernel<8>, dim3(a.nsplit, a.nrt, Hkv), dim3(512), stream, a);
    if (e != hipSuccess || a.nsplit == 1) return e;
    a.cng = 1;
    while (a.cng < 8 && a.cng * 8 < a.nsplit) a.cng *= 2;
    const int rows_wg = 8 / a.cng;
    return launch(tree_attn_combine_kernel, dim3((Hkv * a.R + rows_wg - 1) / rows_wg), dim3(256), stream, a);
}

}  // namespace w4
