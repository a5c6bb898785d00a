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
// with the running max and sum of every row, and the splits are merged
// (log-sum-exp) either by tree_attn_combine_kernel, a second launch, or by
// the last workgroup of each tile to finish (merge_tile): the partial results
// then go out as device-coherent stores, every thread's stores retire, one
// thread counts the workgroup in on the tile's arrival counter, and the
// workgroup that brings the count to the number of splits reads the others'
// results back with device-coherent loads, merges them and sets the counter
// to zero again for the next call (so no clearing launch, and a captured
// call replays).  Nothing ever waits for another workgroup.
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
constexpr int kKT = kChunk / 16;               // 16-key score tiles per chunk
constexpr int kKP = kChunk / 32;               // 32-key value-product steps per chunk
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
    uint32_t* arrive;    // [nrt][Hkv] arrival counters (fused merge)
    int M, L, Hq, Hkv, G, R, T, nrt;
    int nchunks, nsplit, cng;  // cng: thread groups per row in the merge launch
    int fused;                 // the last workgroup of a tile merges its splits
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

// Device-coherent (agent scope) stores and loads of the fused merge: they
// reach or read the level that every XCD shares, past the XCD's own L2.
typedef __attribute__((address_space(1))) uint32_t gu32;
typedef __attribute__((address_space(1))) uint64_t gu64;
__device__ __forceinline__ void store_agent(float* p, float v) {
    __hip_atomic_store((gu32*)p, __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(float* p, f32x4 v) {  // as two 8-byte halves
    __hip_atomic_store((gu64*)p, (uint64_t)__float_as_uint(v[0]) | ((uint64_t)__float_as_uint(v[1]) << 32),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store((gu64*)(p + 2), (uint64_t)__float_as_uint(v[2]) | ((uint64_t)__float_as_uint(v[3]) << 32),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// (a uniform base and a 32-bit byte offset: the workspace is below 4 GB)
__device__ __forceinline__ float load_agent(const float* base, uint32_t off) {
    return __uint_as_float(__hip_atomic_load((const gu32*)((const char*)base + off), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT));
}
// two float pairs, 256 bytes apart
__device__ __forceinline__ f32x4 load_agent2x2(const float* base, uint32_t off) {
    const char* p = (const char*)base + off;
    const uint64_t lo = __hip_atomic_load((const gu64*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t hi = __hip_atomic_load((const gu64*)(p + 256), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return f32x4{__uint_as_float((uint32_t)lo), __uint_as_float((uint32_t)(lo >> 32)), __uint_as_float((uint32_t)hi),
                 __uint_as_float((uint32_t)(hi >> 32))};
}

// The fused merge of rows [r0, r0 + 16W) of key/value head g (the tile's
// real rows): out = sum_s 2^(m_s - m) O_s / sum_s 2^(m_s - m) l_s over the
// splits s.  Thread (rg, c) = (tid / 32, tid % 32) takes head-dim values 2c,
// 2c + 1, 64 + 2c and 65 + 2c of rows r0 + rg + 2W p (so each 8-byte load of
// the 32 threads of a row reads 256 contiguous bytes); its (row, split)
// items run row-major, kB of them in flight at once, merged online (running
// max, rescaled sums); a row is written when its last split is in.
template <int W>
__device__ void merge_tile(const TreeArgs& a, int g, int r0, int tid) {
    constexpr int kB = 24;
    const int rg = tid >> 5, c = tid & 31;
    const int nr = min(16 * W, a.R - r0);
    const int S = a.nsplit;
    const int npair = rg < nr ? (nr - rg + 2 * W - 1) / (2 * W) : 0;
    const int n = npair * S;
    const uint32_t plane = (uint32_t)a.Hkv * a.R;
    const uint32_t row0 = (uint32_t)g * a.R + r0 + rg;  // (head, row) index of pair 0
    int p = 0, s = 0;  // the next item merged
    float mx = -INFINITY, den = 0.0f;
    f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int k0 = 0; k0 < n; k0 += kB) {
        float mv[kB], lv[kB];
        f32x4 ov[kB];
        int pp = p, ss = s;
#pragma unroll
        for (int b = 0; b < kB; ++b) {
            if (k0 + b < n) {
                const uint32_t idx = ss * plane + row0 + 2 * W * pp;
                mv[b] = load_agent(a.mpart, 4 * idx);
                lv[b] = load_agent(a.lpart, 4 * idx);
                ov[b] = load_agent2x2(a.opart, 4 * (idx * kHd + 2 * c));
            }
            if (++ss == S) {
                ss = 0;
                ++pp;
            }
        }
#pragma unroll
        for (int b = 0; b < kB; ++b) {
            if (k0 + b >= n) continue;
            const float nm = fmaxf(mx, mv[b]);
            if (nm != -INFINITY) {
                const float f = exp2_hw(mx - nm), w = exp2_hw(mv[b] - nm);
                acc = acc * f + ov[b] * w;
                den = den * f + lv[b] * w;
                mx = nm;
            }
            if (++s == S) {
                const int r = r0 + rg + 2 * W * p;
                const int tok = r / a.G, head = g * a.G + r % a.G;
                const f32x4 v = den > 0.0f ? acc * (1.0f / den) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                float* const op = a.out + ((size_t)tok * a.Hq + head) * kHd + 2 * c;
                *(float2*)op = make_float2(v[0], v[1]);
                *(float2*)(op + 64) = make_float2(v[2], v[3]);
                s = 0;
                ++p;
                mx = -INFINITY;
                den = 0.0f;
                acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            }
        }
    }
}

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
    // lq of keys lt + 4W r (r < kChunk/4W) and of the value key pairs lt + 4W i
    // (i < kChunk/8W).
    static_assert(W == 4 || W == 8, "4 or 8 waves per workgroup");
    constexpr int KI = kChunk / (4 * W), VI = kChunk / (8 * W), TS = 4 * W;  // TS: thread rows (lt) per workgroup
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
        // scores of the chunk's 16-key tiles
        f32x4 s[kKT];
#pragma unroll
        for (int kt = 0; kt < kKT; ++kt) {
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
            for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) cm = fmaxf(cm, s[kt][r]);
            m_new = fmaxf(m_run, row_max(cm) * a.c);
            alpha = exp2_hw(m_run - m_new);
#pragma unroll
            for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) s[kt][r] = exp2_hw(fmaf(s[kt][r], a.c, -m_new));
        } else {
            float cm = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < kKT; ++kt)
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
            for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) s[kt][r] = none ? 0.0f : exp2_hw(s[kt][r] - m_new);
        }
        // the lane's share of the row sum (the four shares are added at the end)
        float ls = 0.0f;
#pragma unroll
        for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) ls += s[kt][r];
        l_run = l_run * alpha + ls;
        m_run = m_new;
        if (__any(alpha != 1.0f)) {  // the running max moved for some row of the wave
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) oacc[dt] *= alpha;
        }
        // O^T += V^T P^T over the chunk's 32-key steps
#pragma unroll
        for (int kp = 0; kp < kKP; ++kp) {
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
    const size_t base = (size_t)split * plane + (size_t)g * a.R + row;
    float* op = a.opart + base * kHd + 4 * o;
    if (!a.fused) {
        if (row_ok) {
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) *(f32x4*)(op + 16 * dt) = oacc[dt];
            if (o == 0) {
                a.mpart[base] = m_run;
                a.lpart[base] = l_run;
            }
        }
        return;
    }
    if (row_ok) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) store_agent(op + 16 * dt, oacc[dt]);
        if (o == 0) {
            store_agent(a.mpart + base, m_run);
            store_agent(a.lpart + base, l_run);
        }
    }
    // every thread's partial results retire before the workgroup counts in
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    __shared__ uint32_t last;
    uint32_t* const cnt = a.arrive + (size_t)rt * a.Hkv + g;
    if (tid == 0)
        last = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)a.nsplit - 1;
    __syncthreads();
    if (!last) return;
    asm volatile("" ::: "memory");
    // every split of the tile has counted in: merge, and clear the counter
    if (tid == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    merge_tile<W>(a, g, rt * kRowsWg, tid);
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

constexpr size_t kFusedMergeBytes = 72 << 10;  // default limit of a tile's partials for the in-kernel merge
constexpr long long kOneChunkMaxWgs = 288;       // most workgroups of four-wave tiles at one chunk per split

}  // namespace

int tree_attn_plan(int M, int L, int Hq, int Hkv, int merge, int* nsplit_out, int* merge_used, size_t* ws_bytes) {
    const int G = Hq / Hkv, R = M * G, T = L + M;
    const int nchunks = (T + kChunk - 1) / kChunk;
    const int W = tree_waves(R), rows_wg = 16 * W;
    const int nrt = (R + rows_wg - 1) / rows_wg;
    const int tiles = nrt * Hkv;
    // workgroups at once: two of four waves per CU (LDS), one of eight
    // (registers).  Chunks per split: at least two (a workgroup overlaps a
    // chunk's loads with the previous chunk's work), else the fewest that
    // keep to one such round; then at most kTreeMaxSplits splits and what
    // the workspace holds.  Four-wave tiles take one chunk per split while
    // that keeps to about one workgroup per CU (measured with 64 query heads
    // over 8, M = 1 and 2: 0.5-0.9 us faster up to L = 2048, where it makes
    // 264 workgroups; at L = 4096, 520 workgroups, 2 us slower).
    const long long slots = W == 4 ? 512 : 256;
    const int cps_min = W == 4 && (long long)nchunks * tiles <= kOneChunkMaxWgs ? 1 : 2;
    const int cps = std::max(cps_min, (int)(((long long)nchunks * tiles + slots - 1) / slots));
    int nsplit = std::max(1, std::min(kTreeMaxSplits, (nchunks + cps - 1) / cps));
    while (nsplit > 1 && kTreeCounterBytes + partial_bytes(nsplit, Hkv, R) > kTreeWorkspaceBytes) --nsplit;
    if ((size_t)tiles * sizeof(uint32_t) > kTreeCounterBytes) return -1;
    // The merge in the last workgroup of a tile costs a chain of
    // device-coherent round trips (every split's stores acknowledged, the
    // count, the loads of the partials: about 4 us with almost nothing to
    // merge) and then pulls every split's partial rows of the tile through
    // one CU, at 20-30 GB/s; a second launch costs 4.5-7 us but spreads the
    // merge over the chip.  By default the last workgroup merges only
    // four-wave tiles (at most 16 rows) whose partials come to 72 KiB at
    // most (measured with 64 query heads over 8 on these plans: M = 1 and L up
    // to 1024, M = 2 and L up to 256: 0.4-1.4 us per call faster, slower
    // everywhere else).
    int used = kTreeMergeAuto;
    if (nsplit > 1) {
        const size_t tile_bytes = (size_t)nsplit * std::min(R, rows_wg) * (kHd + 2) * sizeof(float);
        used = merge == kTreeMergeLaunch || merge == kTreeMergeLast ? merge
               : W == 4 && tile_bytes <= kFusedMergeBytes       ? kTreeMergeLast
                                                                 : kTreeMergeLaunch;
    }
    if (nsplit_out) *nsplit_out = nsplit;
    if (merge_used) *merge_used = used;
    if (ws_bytes) *ws_bytes = nsplit > 1 ? kTreeCounterBytes + partial_bytes(nsplit, Hkv, R) : 0;
    return 0;
}

hipError_t launch_tree_attn(const uint16_t* q, const uint16_t* kc, const uint16_t* vc, const uint16_t* kd,
                            const uint16_t* vd, const uint64_t* masks, int M, int L, int Hq, int Hkv, float scale,
                            int merge, float* out, void* ws, hipStream_t stream) {
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
    int used = 0;
    if (tree_attn_plan(M, L, Hq, Hkv, merge, &a.nsplit, &used, nullptr) != 0) return hipErrorInvalidValue;
    a.fused = used == kTreeMergeLast;
    a.c = scale * kLog2e;
    const size_t plane = (size_t)a.nsplit * Hkv * a.R;
    a.arrive = (uint32_t*)ws;
    a.opart = (float*)((char*)ws + kTreeCounterBytes);
    a.mpart = a.opart + plane * kHd;
    a.lpart = a.mpart + plane;
    a.out = out;
    hipError_t e = W == 4 ? launch(tree_attn_kernel<4>, dim3(a.nsplit, a.nrt, Hkv), dim3(256), stream, a)
                          : launch(tree_attn_kernel<8>, dim3(a.nsplit, a.nrt, Hkv), dim3(512), stream, a);
    if (e != hipSuccess || a.nsplit == 1 || a.fused) return e;
    a.cng = 1;
    while (a.cng < 8 && a.cng * 8 < a.nsplit) a.cng *= 2;
    const int rows_wg = 8 / a.cng;
    return launch(tree_attn_combine_kernel, dim3((Hkv * a.R + rows_wg - 1) / rows_wg), dim3(256), stream, a);
}

}  // namespace w4
