// HIP kernels of the W4A16 verify linear for gfx950 (CDNA4).
//
// The operation (a weight-only 4-bit linear evaluated over the M tokens of a
// speculative-decoding verify pass; "Speculative Decoding Meets
// Quantization", Abstract, and the ordoresearch.ai review, "Research
// Landscape") is
//     y[m, n] = sum_G s[G, n] * sum_{k in G} x[m, k] * (q[k, n] - z[G, n]).
// The pages call this inference memory-bound; at M <= 64 the 0.52 bytes of
// packed weight per multiply-add dominate every other stream, so every kernel
// here is built around one coalesced pass over the packed weights.
//
// Tile layout (written by w4_repack): a chunk is 64 output columns; for each
// chunk c and k-block kb (32 k) the 64 lanes of a wave read 1 KB, 16 bytes
// per lane.  Lane l's word j carries the 8 codes of column 64c + 16j + l%16
// at k = 32kb + 8(l/16) + e.  That is exactly the B operand of a
// v_mfma_f32_16x16x32_bf16 for n-tile j, so one 128-bit load feeds four
// MFMAs that share one A operand (the activation tile).
//
// Exact operands.  Code e sits at nibble e/2 (even e) or 4 + (e-1)/2 (odd e)
// and the word is stored rotated left by 3 bits, so that
//     rotr(word, 4d) & 0x00780078 | 0x41804180
// is the bf16 pair (16 + q[2d], 16 + q[2d+1]): each code lands in the top
// four mantissa bits of a bf16 whose exponent is that of 16.0, a step of
// exactly 1.  The kernels accumulate x . (16 + q) per group in fp32 and
// subtract (16 + z) * sum(x) per group before the fp32 group scale, so no
// weight is ever rounded.  The bias (16, the smallest a 4-bit code in a
// 7-bit bf16 mantissa allows) is what the subtraction cancels: the fp32
// partial sums carry about (16 + q) * sum|x| instead of |x . (q - z)|.
#include "w4_internal.h"
#include "w4_device.h"

#include <algorithm>
#include <cmath>
#include <mutex>

namespace w4 {

// ---------------------------------------------------------------------------
// repack: canonical -> tile layout (offline, not timed)
// ---------------------------------------------------------------------------

// Moves canonical nibble e (k offset e) to tile nibble e/2 (even e) or
// 4 + (e-1)/2 (odd e), then rotates the word left by 3 bits (see
// unpack_biased).
__device__ __forceinline__ uint32_t to_tile_nibbles(uint32_t w) {
    uint32_t out = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int p = (e & 1) ? 4 + (e >> 1) : (e >> 1);
        out |= ((w >> (4 * e)) & 15u) << (4 * p);
    }
    return (out << 3) | (out >> 29);
}

// One thread per tile word.  Thread order (c, kb, o, j, t) keeps canonical
// reads coalesced along n.
__global__ void repack_qweight_kernel(const int32_t* __restrict__ qweight, int N, int K, uint32_t* __restrict__ out,
                                      size_t total) {
    const int KB = K / kKBlock;
    for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (size_t)gridDim.x * blockDim.x) {
        const int t = (int)(idx & 15);
        const int j = (int)((idx >> 4) & 3);
        const int o = (int)((idx >> 6) & 3);
        const size_t rest = idx >> 8;
        const int kb = (int)(rest % KB);
        const size_t c = rest / KB;
        const size_t n = c * kChunkN + 16 * j + t;
        uint32_t w = 0;
        if (n < (size_t)N) w = (uint32_t)qweight[(size_t)(4 * kb + o) * N + n];
        const int lane = o * 16 + t;
        out[((c * KB + kb) * 64 + lane) * 4 + j] = to_tile_nibbles(w);
    }
}

// A (group, column) whose every code equals its zero point holds only zero
// weights, s (q - z) = 0 for any s; its scale is stored as 0.  The kernels
// form s * (sum x (16 + q) - (16 + z) sum x), and the two sums of such a
// group cancel exactly only when 16 + z is a power of two (z = 0): with the
// scale 0 the group adds exactly 0 for every z, so a column of zero weights
// gives exactly 0 as the contract requires (its bound is 0 there), also for
// the z = 8 a symmetric quantiser writes.  Codes and zero points are stored
// unchanged.
__global__ void repack_scales_kernel(const int32_t* __restrict__ qweight, const uint16_t* __restrict__ scales,
                                     const int32_t* __restrict__ zeros, int N, int K, uint16_t* __restrict__ s_out,
                                     uint16_t* __restrict__ z_out, size_t total) {
    const int G = K / kGroup;
    // one thread per (c, G, t)
    for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (size_t)gridDim.x * blockDim.x) {
        const int t = (int)(idx & 15);
        const size_t rest = idx >> 4;
        const int g = (int)(rest % G);
        const size_t c = rest / G;
        uint32_t zw = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const size_t n = c * kChunkN + 16 * j + t;
            uint16_t s = 0;
            uint32_t z = 0;
            if (n < (size_t)N) {
                s = scales[(size_t)g * N + n];
                z = ((uint32_t)zeros[(size_t)g * (N / 8) + n / 8] >> (4 * (n % 8))) & 15u;
                bool flat = true;  // every code of the group equals z
                for (int i = 0; i < kGroup / 8; ++i)
                    flat &= (uint32_t)qweight[((size_t)g * (kGroup / 8) + i) * N + n] == z * 0x11111111u;
                if (flat) s = 0;
            }
            s_out[idx * 4 + j] = s;
            zw |= z << (4 * j);
        }
        z_out[idx] = (uint16_t)zw;
    }
}

// ---------------------------------------------------------------------------
// unpack (test only): tile layout -> canonical bytes through unpack_biased
// ---------------------------------------------------------------------------

__global__ void unpack_qweight_kernel(const uint32_t* __restrict__ qt, int N, int K, uint8_t* __restrict__ q_out,
                                      size_t total, uint32_t mask, uint32_t magic) {
    const int KB = K / kKBlock;
    for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (size_t)gridDim.x * blockDim.x) {
        const int j = (int)(idx & 3);
        const int lane = (int)((idx >> 2) & 63);
        const size_t rest = idx >> 8;
        const int kb = (int)(rest % KB);
        const size_t c = rest / KB;
        const size_t n = c * kChunkN + 16 * j + (lane & 15);
        if (n >= (size_t)N) continue;
        const u32x4 b = unpack_biased(qt[idx], mask, magic);
        const size_t k0 = (size_t)kb * kKBlock + 8 * (lane >> 4);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const float lo = bf16_bits_to_f32(b[d] & 0xFFFFu) - kCodeBias;
            const float hi = bf16_bits_to_f32(b[d] >> 16) - kCodeBias;
            q_out[(k0 + 2 * d) * N + n] = (uint8_t)lo;
            q_out[(k0 + 2 * d + 1) * N + n] = (uint8_t)hi;
        }
    }
}

__global__ void unpack_zeros_kernel(const uint16_t* __restrict__ zt, int N, int K, uint8_t* __restrict__ z_out,
                                    size_t total) {
    const int G = K / kGroup;
    for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (size_t)gridDim.x * blockDim.x) {
        const int t = (int)(idx & 15);
        const size_t rest = idx >> 4;
        const int g = (int)(rest % G);
        const size_t c = rest / G;
        const uint32_t zw = zt[idx];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const size_t n = c * kChunkN + 16 * j + t;
            if (n < (size_t)N) z_out[(size_t)g * N + n] = (uint8_t)(biased_zero(zw, j) - kCodeBias);
        }
    }
}

// ---------------------------------------------------------------------------
// verify linear: shared pieces
// ---------------------------------------------------------------------------

struct LinearArgs {
    const uint16_t* x;
    const u32x4* qt;
    const uint2* st;
    const uint16_t* zt;
    float* y;        // fp32 output when not null, and/or
    uint16_t* yb;    // bf16 output (round to nearest even) when not null
    float alpha;     // output scale (1 for the plain linear)
    float* ws;
    int M, N, K;
    int ldx;         // elements between consecutive rows of x (>= K)
    int NC, KB, G;
    int gps, splits, ntiles;
    int kw;          // waves of a workgroup that split one chunk's K range (1: one chunk per wave)
    int rs;          // row slices of the LDS kernel (workgroups along M, 16 MB rows each)
    uint32_t mask;   // 0x00780078 (see unpack_biased)
    uint32_t magic;  // 0x41804180: bf16 16.0 in both halves
};

// Final value of y[i] (unsplit K), scaled by alpha: fp32 and/or bf16 (the
// bf16 epilogue).  alpha = 1 leaves every value's bits unchanged.
__device__ __forceinline__ void store_y(const LinearArgs& a, size_t i, float v) {
    v *= a.alpha;
    if (a.y) a.y[i] = v;
    if (a.yb) a.yb[i] = f32_to_bf16_rne(v);
}

// Weight ring.  A wave keeps kRing groups of weights (4 x 16 bytes per lane
// each, plus the group's scales and zeros) in flight ahead of the group it
// computes.  Every slot is reloaded unconditionally right after its group is
// consumed -- past the wave's last group the address is clamped to that group
// (an L2 hit) -- so the compiler never has to merge an old and a new value of
// a slot, which would force it to wait for the load it just issued.
template <int R>
struct WeightRing {
    u32x4 w[R][4];
    uint2 s[R];
    uint32_t z[R];
};

struct WaveStream {
    const u32x4* wp;    // first weight word of the wave's first group (lane offset applied)
    const uint2* sp;    // scales of the first group (column offset applied)
    const uint16_t* zp; // zeros of the first group
};

template <int R>
__device__ __forceinline__ void ring_load(WeightRing<R>& ring, int slot, const WaveStream& ws, int gl) {
    // keep the reload after the slot's last use: if the scheduler hoisted it,
    // old and new values would be live together and the register allocator
    // would insert copies that wait for the load
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) ring.w[slot][kk] = ws.wp[(gl * 4 + kk) * 64];
    ring.s[slot] = ws.sp[gl * 16];
    ring.z[slot] = ws.zp[gl * 16];
}

__device__ __forceinline__ WaveStream wave_stream(const LinearArgs& a, int c, int g0, int lane) {
    WaveStream ws;
    ws.wp = a.qt + ((size_t)c * a.KB + (size_t)g0 * 4) * 64 + lane;
    ws.sp = a.st + ((size_t)c * a.G + g0) * 16 + (lane & 15);
    ws.zp = a.zt + ((size_t)c * a.G + g0) * 16 + (lane & 15);
    return ws;
}

// The work of one wave of the streaming kernels (M <= 16).  With kw == 1 a
// workgroup covers four chunks, one per wave, over the groups of its K split;
// with kw > 1 it covers one chunk and its kw waves split the split's groups
// between them (contiguous, as even as possible), to be summed in LDS.
struct WaveWork {
    int split, c, kidx, g0, ng;
};

__device__ __forceinline__ WaveWork wave_work(const LinearArgs& a, int wave) {
    WaveWork w;
    w.split = blockIdx.x / a.ntiles;
    const int tile = blockIdx.x - w.split * a.ntiles;
    const int gs = w.split * a.gps;
    const int gwg = min(a.G, gs + a.gps) - gs;
    w.kidx = a.kw == 1 ? 0 : wave;
    w.c = a.kw == 1 ? tile * kWaves + wave : tile;
    const int lo = gwg * w.kidx / a.kw, hi = gwg * (w.kidx + 1) / a.kw;
    w.g0 = gs + lo;
    w.ng = hi - lo;  // >= 1: the planner gives every wave a group
    return w;
}

// ---------------------------------------------------------------------------
// M = 1: VALU GEMV (bf16 dot2, fp32 accumulation, cross-lane shuffles)
// ---------------------------------------------------------------------------
//
// Lane (o = l/16, t = l%16) accumulates, for its 4 columns 64c + 16j + t, the
// k of octet o in every k-block.  Its activation octets come straight from
// global memory (x is only 2K bytes and stays in L1/L2) in the same load ring
// as the weights, so a wave never waits on LDS or a barrier, and the
// per-group sum of those octets (the zero-point term) is the lane's own.  The
// four octet lanes of a column are summed with two xor-shuffles at the end.



// Groups of loads each wave keeps in flight (a slot is 4 weight words, the
// activation pieces, one scale word and one zero word per lane; the total
// stays under the 63 outstanding loads a wave can track).
constexpr int kRingGemv = 4;
constexpr int kRingDirect1 = 4;

template <int R>
__global__ __launch_bounds__(kMaxThreads) void w4a16_gemv_kernel(LinearArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const WaveWork wk = wave_work(a, wave);
    const int split = wk.split, c = wk.c, g0 = wk.g0, ng = wk.ng;
    const int o = lane >> 4, t = lane & 15;
    const uint32_t mask = a.mask, magic = to_vgpr(a.magic);
    // waves past the last chunk stream the last chunk again (never stored):
    // branch-free loads keep the compiler's wait counts exact
    const WaveStream ws = wave_stream(a, min(c, a.NC - 1), g0, lane);
    const u32x4* xp = (const u32x4*)(a.x + (size_t)g0 * kGroup + 8 * o);  // 16-byte units

    u32x4 rw[R][4], rx[R][4];
    uint2 rs[R];
    uint32_t rz[R];
    auto load = [&](int d, int gl) {
        __builtin_amdgcn_sched_barrier(0);  // keep the reload after the slot's last use
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) rw[d][kk] = load_stream(ws.wp + (gl * 4 + kk) * 64);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) rx[d][kk] = xp[gl * 16 + kk * 4];
        rs[d] = load_stream(ws.sp + gl * 16);
        rz[d] = load_stream(ws.zp + gl * 16);
    };

    float yv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int d = 0; d < R; ++d) load(d, min(d, ng - 1));
    for (int gb = 0; gb < ng; gb += R) {
#pragma unroll
        for (int d = 0; d < R; ++d) {
            const int gl = gb + d;
            if (gl < ng) {
                float acc[4];
                float xs = 0.0f;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const u32x4 xa = rx[d][kk];
                    const uint32_t x0 = xa[0], x1 = xa[1], x2 = xa[2], x3 = xa[3];
                    xs = dot2(x0, kOnesBf16x2, xs);
                    xs = dot2(x1, kOnesBf16x2, xs);
                    xs = dot2(x2, kOnesBf16x2, xs);
                    xs = dot2(x3, kOnesBf16x2, xs);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const u32x4 b = unpack_biased(rw[d][kk][j], mask, magic);
                        float s0 = kk == 0 ? 0.0f : acc[j];
                        s0 = dot2(b[0], x0, s0);
                        s0 = dot2(b[1], x1, s0);
                        s0 = dot2(b[2], x2, s0);
                        s0 = dot2(b[3], x3, s0);
                        acc[j] = s0;
                    }
                }
                float sj[4];
                decode_scales(rs[d], sj);
                const uint32_t zw = rz[d];
#pragma unroll
                for (int j = 0; j < 4; ++j) yv[j] = fmaf(sj[j], fmaf(-biased_zero(zw, j), xs, acc[j]), yv[j]);
            }
            load(d, min(gl + R, ng - 1));
        }
    }
    // sum the four octet lanes of each column
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        yv[j] += __shfl_xor(yv[j], 16);
        yv[j] += __shfl_xor(yv[j], 32);
    }
    if (a.kw > 1) {
        // the K parts of the chunk, summed by wave 0 in wave order
        __shared__ float red[kMaxWaves][kChunkN];
        if (o == 0)
#pragma unroll
            for (int j = 0; j < 4; ++j) red[wk.kidx][4 * t + j] = yv[j];
        __syncthreads();
        if (wk.kidx == 0)
            for (int k2 = 1; k2 < a.kw; ++k2)
#pragma unroll
                for (int j = 0; j < 4; ++j) yv[j] += red[k2][4 * t + j];
    }
    if (c < a.NC && o == 0 && wk.kidx == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = c * kChunkN + 16 * j + t;
            if (n < a.N) {
                if (a.splits == 1)
                    store_y(a, n, yv[j]);
                else
                    store_partial(a.ws + (size_t)split * a.NC * kChunkN + n, yv[j]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// M = 2..16: bf16 MFMA with activations loaded straight into A operands
// ---------------------------------------------------------------------------
//
// For small M the activation rows are tiny and L1/L2-resident, so each lane
// loads its own A operand (row 16mb + l%16, k-octet l/16 of each k-block)
// from global memory in the same ring as the weights: no LDS, no barriers.
// Rows past M load row M - 1 again: an MFMA output row depends on its own A
// row only, and rows past M are never stored, so they need no zeroing.  One
// extra MFMA per k-block against an all-ones B operand yields the
// per-(row, group) sums of x that the zero-point term needs, already in the
// result layout (rows 4(l/16) + r).

template <int MB, int R>
__global__ __launch_bounds__(kMaxThreads) void w4a16_mfma_direct_kernel(LinearArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const WaveWork wk = wave_work(a, wave);
    const int split = wk.split, c = wk.c, g0 = wk.g0, ng = wk.ng;
    const int o = lane >> 4, t = lane & 15;
    const uint32_t mask = a.mask, magic = to_vgpr(a.magic);
    const WaveStream ws = wave_stream(a, min(c, a.NC - 1), g0, lane);
    const u32x4* xp[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int row = 16 * mb + t;
        xp[mb] = (const u32x4*)(a.x + (size_t)min(row, a.M - 1) * a.ldx + (size_t)g0 * kGroup + 8 * o);
    }
    const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{kOnesBf16x2, kOnesBf16x2, kOnesBf16x2, kOnesBf16x2});

    u32x4 rw[R][4], rx[R][4][MB];
    uint2 rs[R];
    uint32_t rz[R];
    auto load = [&](int d, int gl) {
        __builtin_amdgcn_sched_barrier(0);  // keep the reload after the slot's last use
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) rw[d][kk] = load_stream(ws.wp + (gl * 4 + kk) * 64);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) rx[d][kk][mb] = xp[mb][gl * 16 + kk * 4];
        rs[d] = load_stream(ws.sp + gl * 16);
        rz[d] = load_stream(ws.zp + gl * 16);
    };

    f32x4 yv[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) yv[mb][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // A group's scale epilogue runs after the next group's MFMAs are issued:
    // the VALU reads an MFMA result only once the MFMA has finished, which
    // takes far longer than forwarding it to a dependent MFMA, so reading a
    // group's accumulators right after its last MFMA stalled the wave every
    // group.  Two sets of accumulators (and of the group's scales and zeros)
    // alternate with the group's parity, which is the ring slot's (R even).
    // The epilogues still add into yv in group order.
    static_assert(R % 2 == 0, "accumulator sets alternate with the ring slot");
    f32x4 acc[2][MB][4], accx[2][MB];
    float sjh[2][4];
    uint32_t zwh[2];
    auto epilogue = [&](int b) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float cz = biased_zero(zwh[b], j);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    yv[mb][j][r] = fmaf(sjh[b][j], fmaf(-cz, accx[b][mb][r], acc[b][mb][j][r]), yv[mb][j][r]);
            }
    };

#pragma unroll
    for (int d = 0; d < R; ++d) load(d, min(d, ng - 1));
    for (int gb = 0; gb < ng; gb += R) {
#pragma unroll
        for (int d = 0; d < R; ++d) {
            const int gl = gb + d;
            if (gl < ng) {
                const int b = d & 1;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    bf16x8 av[MB];
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) av[mb] = __builtin_bit_cast(bf16x8, rx[d][kk][mb]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const u32x4 braw = unpack_biased(rw[d][kk][j], mask, magic);
                        const bf16x8 bv = __builtin_bit_cast(bf16x8, braw);
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb)
                            acc[b][mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                av[mb], bv, kk == 0 ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : acc[b][mb][j], 0, 0, 0);
                    }
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
                        accx[b][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            av[mb], ones, kk == 0 ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : accx[b][mb], 0, 0, 0);
                }
                decode_scales(rs[d], sjh[b]);
                zwh[b] = rz[d];
                if (gl > 0) epilogue(b ^ 1);  // the previous group's
            }
            load(d, min(gl + R, ng - 1));
        }
    }
    if (ng > 0) {  // the last group's epilogue
        if ((ng - 1) & 1)
            epilogue(1);
        else
            epilogue(0);
    }

    if (a.kw > 1) {
        // the K parts of the chunk, summed by wave 0 in wave order
        static_assert(MB == 1, "the LDS sum holds one row block");
        __shared__ f32x4 red[kMaxWaves - 1][4][64];
        if (wk.kidx > 0)
#pragma unroll
            for (int j = 0; j < 4; ++j) red[wk.kidx - 1][j][lane] = yv[0][j];
        __syncthreads();
        if (wk.kidx == 0)
            for (int k2 = 1; k2 < a.kw; ++k2)
#pragma unroll
                for (int j = 0; j < 4; ++j) yv[0][j] += red[k2 - 1][j][lane];
    }
    if (c < a.NC && wk.kidx == 0) {
        const size_t npad = (size_t)a.NC * kChunkN;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = c * kChunkN + 16 * j + t;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = 16 * mb + 4 * o + r;
                    if (m < a.M && n < a.N) {
                        if (a.splits == 1)
                            store_y(a, (size_t)m * a.N + n, yv[mb][j][r]);
                        else
                            store_partial(a.ws + ((size_t)split * a.M + m) * npad + n, yv[mb][j][r]);
                    }
                }
            }
    }
}

// ---------------------------------------------------------------------------
// M = 17..64 (and M = 15, 16 on linears of 4096 or more columns): bf16
// MFMA, one wave per 64-column chunk over all rows, activations copied into
// a three-deep LDS ring by the LDS DMA path
// ---------------------------------------------------------------------------
//
// Each wave owns one chunk and every row block of 16 of its workgroup's row
// slice (all rows, or, on narrow linears, MB row blocks starting at row
// 16 MB * slice), so each unpacked weight feeds MB MFMAs and each A operand
// read from LDS feeds four: the LDS traffic is four bytes of activations per
// byte of weights at M = 64.  A workgroup
// holds WV = 4 or 8 chunks (the planner's choice per shape) that share one
// activation copy; two waves per SIMD (two 4-wave workgroups per CU, or one
// 8-wave workgroup) overlap one wave's MFMAs with the other's unpack and
// epilogue VALU work; a wave raises its priority while it issues MFMAs, so
// the matrix pipe is fed first whenever both waves are ready.
//
// Activations never pass through VGPRs: global_load_lds_dwordx4 writes a
// lane's 16 bytes straight to byte 16*lane of a 1 KB LDS line, and the
// global address of each lane is free, so the line is filled in a
// bank-swizzled order: row r of a group keeps k-octet q at 16-byte slot
// q ^ (r & 15).  A wave's A-operand read (rows 16mb + l%16, octet 4kk + l/16)
// then touches sixteen distinct 16-byte slots of a 256-byte bank window in
// every sixteen lanes.
//
// The per-(row, group) activation sums of the zero-point term come from one
// extra MFMA per k-block against an all-ones B operand: wave w computes them
// for row block w one group ahead and publishes them through LDS.
//
// Pipeline per group g (one workgroup barrier):
//   MFMAs of group g from buffer g%3 and weight ring slot g%3, the last
//   k-block row block by row block;
//   epilogue of each row block two row blocks after its last MFMA (an MFMA
//   result takes far longer to become readable by the VALU than by a
//   dependent MFMA), the sums of group g+1 in between;
//   wait for this wave's DMA of group g+2, then barrier;
//   DMA of group g+3 into buffer g%3, then the weight loads of group g+3
//   into ring slot g%3.
// Every buffer is rewritten only after the barrier that follows its last
// read.  The DMA is issued from inline asm: the compiler's wait-count pass
// treats LDS DMA and register loads in flight together as possibly out of
// order and would wait for every load (vmcnt(0)) before each use of the
// weight ring.  Loads retire in issue order, so the explicit wait for the
// DMA of group g+2 needs only the ring loads issued after it to stay in
// flight, and the compiler's own waits for ring data (which do not count the
// hidden DMA) can only wait longer than needed, never too little.

constexpr int kLdsRing = 3;  // activation buffers, sum slots and weight ring depth

__host__ __device__ constexpr int lds_ring_xbuf(int mb) { return 16 * mb * kGroup * 2; }
__host__ __device__ constexpr int lds_ring_bytes(int mb) { return kLdsRing * (lds_ring_xbuf(mb) + 16 * mb * 4); }

// Wait until at most N vector memory loads of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int MB, int WV>
__global__ __launch_bounds__(64 * WV) __attribute__((amdgpu_waves_per_eu(2, 2))) void w4a16_mfma_lds_kernel(LinearArgs a) {
    static_assert(WV == 4 || WV == 8, "four or eight chunks per workgroup");
    constexpr int XD = (4 * MB + WV - 1) / WV;  // activation lines (4 rows each) this wave copies per group
    constexpr int R = kLdsRing;
    constexpr int XB = lds_ring_xbuf(MB);  // bytes per activation buffer
    constexpr int XS = R * XB;             // first sum slot
    constexpr int XSS = 16 * MB * 4;       // bytes per sum slot
    constexpr int kRingOps = 6;            // loads per weight ring slot: 4 weight words, scales, zeros
    extern __shared__ __align__(16) char smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // workgroup = (row slice, K split, column tile), the tile fastest
    const int per_slice = a.splits * a.ntiles;
    const int slice = blockIdx.x / per_slice;
    const int split = (blockIdx.x - slice * per_slice) / a.ntiles;
    const int tile = blockIdx.x - slice * per_slice - split * a.ntiles;
    const int g0 = split * a.gps;
    const int ng = min(a.G, g0 + a.gps) - g0;
    const int c = tile * WV + wave;
    const int m0 = slice * 16 * MB;            // first row of this slice
    const int ml = min(a.M - m0, 16 * MB);     // its rows (>= 1)
    const int o = lane >> 4, t = lane & 15;
    const uint32_t mask = a.mask, magic = to_vgpr(a.magic);
    const WaveStream ws = wave_stream(a, min(c, a.NC - 1), g0, lane);
    const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{kOnesBf16x2, kOnesBf16x2, kOnesBf16x2, kOnesBf16x2});

    // DMA sources.  A buffer holds 4 MB lines; wave w fills lines w + WV ii
    // (ii < XD; a line past the last is replaced by the wave's previous one,
    // or with fewer lines than waves by line w % 4MB: a second copy of the
    // same bytes to the same place).  Line i holds rows m0 + 4i..4i+3 of the
    // slice and lane l lands in row 4i + l/16, slot l%16, which holds
    // k-octet (l%16) ^ (row & 15).  Rows past the slice's last repeat it
    // (their results are never stored), groups past the split repeat its
    // last group.
    int xoff[XD], xline[XD];
#pragma unroll
    for (int ii = 0; ii < XD; ++ii) {
        int line = wave + WV * ii;
        if (line >= 4 * MB) line = 4 * MB >= WV ? line - WV : line % (4 * MB);
        xline[ii] = line;
        const int r = 4 * line + o;
        xoff[ii] = (m0 + min(r, ml - 1)) * a.ldx + 8 * (t ^ (r & 15));
    }
    const uint16_t* xg = a.x + (size_t)g0 * kGroup;
    auto issue_x = [&](int buf, int gl) {
        const uint16_t* src = xg + (size_t)min(gl, ng - 1) * kGroup;
#pragma unroll
        for (int ii = 0; ii < XD; ++ii) lds_dma16(src + xoff[ii], smem + buf * XB + 1024 * xline[ii]);
    };

    // A operand of (row block mb, k-block kk) in buffer b: row 16mb + t, octet
    // 4kk + o, at slot (4kk + o) ^ t.  One base per kk; the buffer and the
    // row block are immediate offsets.
    int ab[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) ab[kk] = (16 * t + ((4 * kk + o) ^ t)) * 16;
    auto a_frag = [&](int b, int mb, int kk) -> bf16x8 {
        return __builtin_bit_cast(bf16x8, *(const u32x4*)(smem + ab[kk] + b * XB + mb * 4096));
    };
    // zero-point sums of row block `wave` of the group in buffer b, into sum slot b
    auto compute_xs = [&](int b) {
        if (wave < MB) {
            f32x4 accx = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const bf16x8 av =
                    __builtin_bit_cast(bf16x8, *(const u32x4*)(smem + ab[kk] + wave * 4096 + b * XB));
                accx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, ones, accx, 0, 0, 0);
            }
            // D rows 4o + r of the block; every column holds the same sums
            if (t == 0) *(f32x4*)(smem + XS + b * XSS + (16 * wave + 4 * o) * 4) = accx;
        }
    };

    WeightRing<R> ring;
#pragma unroll
    for (int d = 0; d < R; ++d) {
        issue_x(d, d);
        ring_load(ring, d, ws, min(d, ng - 1));
    }
    // groups 0 and 1 landed: after them only the ring slot of group 1, then
    // the DMA and ring slot of group 2 may still be in flight
    wait_vmcnt<2 * kRingOps + XD>();
    lds_barrier();
    compute_xs(0);
    lds_barrier();

    f32x4 yv[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) yv[mb][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    for (int gb = 0; gb < ng; gb += R) {
#pragma unroll
        for (int d = 0; d < R; ++d) {
            const int gl = gb + d;  // buffer, sum slot and ring slot are all d = gl % 3
            if (gl < ng) {
                __builtin_amdgcn_s_setprio(1);
                f32x4 acc[MB][4];
#pragma unroll
                for (int kk = 0; kk < 3; ++kk) {
                    bf16x8 av[MB];
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) av[mb] = a_frag(d, mb, kk);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const u32x4 braw = unpack_biased(ring.w[d][kk][j], mask, magic);
                        const bf16x8 bv = __builtin_bit_cast(bf16x8, braw);
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb)
                            acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                av[mb], bv, kk == 0 ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : acc[mb][j], 0, 0, 0);
                    }
                }
                __builtin_amdgcn_s_setprio(0);
                float sj[4], cz[4];
                decode_scales(ring.s[d], sj);
#pragma unroll
                for (int j = 0; j < 4; ++j) cz[j] = biased_zero(ring.z[d], j);
                // last k-block row block by row block, so the epilogue of one
                // row block can issue while the MFMAs of the next one run
                bf16x8 bv3[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) bv3[j] = __builtin_bit_cast(bf16x8, unpack_biased(ring.w[d][3][j], mask, magic));
                auto epi = [&](int mb) {
                    const f32x4 xs = *(const f32x4*)(smem + XS + d * XSS + (16 * mb + 4 * o) * 4);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            yv[mb][j][r] = fmaf(sj[j], fmaf(-cz[j], xs[r], acc[mb][j][r]), yv[mb][j][r]);
                };
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const bf16x8 av = a_frag(d, mb, 3);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv3[j], acc[mb][j], 0, 0, 0);
                    if (mb >= 2) epi(mb - 2);
                }
                if (gl + 1 < ng) compute_xs((d + 1) % R);
#pragma unroll
                for (int mb = MB >= 2 ? MB - 2 : 0; mb < MB; ++mb) epi(mb);
                wait_vmcnt<kRingOps>();  // this wave's DMA of group gl+2 (its ring slot may still fly)
                lds_barrier();
                issue_x(d, gl + R);
            }
            ring_load(ring, d, ws, min(gl + R, ng - 1));
        }
    }
    wait_vmcnt<0>();  // no DMA into LDS outlives the loop

    if (c < a.NC) {
        const size_t npad = (size_t)a.NC * kChunkN;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = c * kChunkN + 16 * j + t;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = m0 + 16 * mb + 4 * o + r;
                    if (m - m0 < ml && n < a.N) {
                        if (a.splits == 1)
                            store_y(a, (size_t)m * a.N + n, yv[mb][j][r]);
                        else
                            store_partial(a.ws + ((size_t)split * a.M + m) * npad + n, yv[mb][j][r]);
                    }
                }
            }
    }
}

// ---------------------------------------------------------------------------
// split-K reduction
// ---------------------------------------------------------------------------
//
// With S > 1 every workgroup writes its partial [M x 256] tile to the
// workspace and the sum is a second launch on the same stream (the kernel
// boundary orders and publishes the partial stores).  Measured against the
// alternative -- the last workgroup of a tile to finish sums the tile alone,
// found through a per-tile atomic counter -- it is 1-4 us faster per launch:
// the fix-up chain (counter round trip, then S*M/32 dependent partial loads
// by 256 threads) sits after all the streaming, while the second launch
// spreads the same reads over the chip.  One thread per 4 output columns of a
// row keeps its S partial vectors in flight together (KB >= S loads issued
// before the first add, so the whole sum costs one memory round trip: with
// batches of 8, S = 11..22 took two or three and the launch ~4.5 us even for
// a single workgroup) and adds them in split order (deterministic; the same
// bits for every KB).
template <int KB>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ ws, float* __restrict__ y,
                                                          uint16_t* __restrict__ yb, float alpha, int M, int N,
                                                          int npad, int splits) {
    const int nq = N / 4;
    const size_t total = (size_t)M * nq;
    const size_t plane = (size_t)M * npad;
    for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (size_t)gridDim.x * blockDim.x) {
        const int m = (int)(idx / nq);
        const int n = 4 * (int)(idx - (size_t)m * nq);
        const f32x4* src = (const f32x4*)(ws + (size_t)m * npad + n);
        f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        for (int s0 = 0; s0 < splits; s0 += KB) {
            f32x4 v[KB];
#pragma unroll
            for (int i = 0; i < KB; ++i) v[i] = src[(size_t)min(s0 + i, splits - 1) * (plane / 4)];
#pragma unroll
            for (int i = 0; i < KB; ++i)
                if (s0 + i < splits) acc += v[i];
        }
        const size_t o = (size_t)m * N + n;
        acc *= alpha;
        if (yb) {
            const float a0 = acc[0], a1 = acc[1], a2 = acc[2], a3 = acc[3];
            const uint32_t lo = f32_to_bf16_rne(a0) | ((uint32_t)f32_to_bf16_rne(a1) << 16);
            const uint32_t hi = f32_to_bf16_rne(a2) | ((uint32_t)f32_to_bf16_rne(a3) << 16);
            *(uint2*)(yb + o) = uint2{lo, hi};
        }
        if (y) *(f32x4*)(y + o) = acc;
    }
}

// ---------------------------------------------------------------------------
// small kernels
// ---------------------------------------------------------------------------

__global__ void zero_kernel(float* __restrict__ y, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) y[i] = 0.0f;
}

// Streaming read of a buffer (the HBM read ceiling and the per-linear read
// floor): workgroup b reads the contiguous 1 KB blocks [b*per, (b+1)*per),
// wave w every fourth of them, U 16-byte loads per lane in flight; the last
// workgroup also reads the tail past the last whole block.  Each workgroup
// writes the xor of everything it read to sink[b], so no load can be dropped.
template <int U>
__global__ __launch_bounds__(256) void bench_read_kernel(const u32x4* __restrict__ buf, size_t n16, size_t per,
                                                         uint32_t* __restrict__ sink) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const size_t nblk = n16 / 64;
    const size_t b0 = (size_t)blockIdx.x * per;
    const size_t b1 = min(nblk, b0 + per);
    uint32_t acc = 0;
    size_t b = b0 + wave;
    for (; b + 4 * (U - 1) < b1; b += 4 * U) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(buf + (b + 4 * u) * 64 + lane);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; b < b1; b += 4) {
        const u32x4 v = buf[b * 64 + lane];
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    if (blockIdx.x == gridDim.x - 1 && wave == 0 && nblk * 64 + lane < n16) {
        const u32x4 v = buf[nblk * 64 + lane];
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
    __shared__ uint32_t part[4];
    if (lane == 0) part[wave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

__global__ __launch_bounds__(256) void bench_copy_kernel(u32x4* __restrict__ dst, const u32x4* __restrict__ src,
                                                         size_t n16) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

// ---------------------------------------------------------------------------
// the allocation-free entry point's split-K scratch
// ---------------------------------------------------------------------------
//
// A file-scope device array that every GPU running the library holds from
// module load until the process ends.  In host code its name is only a
// stand-in for the symbol: the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current
// and kept per device; kernels receive that address, never the name.
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

hipError_t noalloc_scratch(Workspace* ws) {
    constexpr int kMaxDev = 64;
    static std::mutex mu;
    static void* addr[kMaxDev] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    ws->partial = (float*)addr[dev];
    ws->partial_bytes = kNoAllocScratchBytes;
    return hipSuccess;
}

// ---------------------------------------------------------------------------
// planning and launches
// ---------------------------------------------------------------------------

static int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

int plan_linear(int M, int N, int K, int kernel, int splits, int kwaves, size_t ws_bytes, Plan* p) {
    if (kernel == kAuto) kernel = (M == 1) ? kGemv : kMfma;
    if (kernel == kGemv && M != 1) return -1;
    if (kwaves < 0 || kwaves > kMaxWaves || (kwaves & (kwaves - 1)) != 0) return -1;
    const int NC = ceil_div(N, kChunkN);
    const int G = K / kGroup;
    const int mb = ceil_div(M, 16);
    // One row block (M <= 16) streams through the direct MFMA kernel, except
    // at M >= 15 on linears of 4096 or more columns, where the LDS kernel's
    // shared activation copy wins (measured at M = 16: q 16.5 -> 13.9 us,
    // lm_head 114.7 -> 103.5, gate 32.9 -> 32.1, down 30.0 -> 29.4; k and v,
    // 1024 columns, and M <= 14 on gate and down are faster direct).
    const bool lds_one_block = M >= 15 && N >= 4096 && kwaves == 0;
    const int variant = kernel == kGemv ? kVarGemv : ((mb == 1 && !lds_one_block) ? kVarDirect : kVarLds);
    int lds_wv = kWaves;  // chunks per workgroup of the M > 16 kernel
    int rs = 1;           // its row slices
    if (variant == kVarLds && kwaves > 1) return -1;
    int kw = 1;
    int S = 1;
    if (variant != kVarLds) {
        // Streaming kernels (M <= 16): the work decomposition (kw waves per
        // chunk, S K splits) of least modelled time.  Model, fitted to
        // MI355X sweeps of every decomposition on the Llama-3-70B shapes:
        // a CU streams at most ~30 GB/s and the chip ~5.8 TB/s; a launch
        // costs ~3 us before the stream runs at rate; a split K adds ~3.5 us
        // (partials, then the reduction launch) plus the partial traffic;
        // waves beyond what the CUs hold at once (12 per CU for the GEMV,
        // 8 for the MFMA kernel) cost ~3 us per extra round.  Ties go to
        // fewer splits, then fewer waves per chunk.  Left to the planner, a
        // chunk gets 1 or 4 waves: with 2 too few loads are in flight per CU
        // (gate at M = 1: 33 us with 2, 27 us with 4), and 8 gained nothing.
        const double bytes = 0.52 * N * (double)K;
        const double red_bytes = (double)M * NC * kChunkN * 8;
        const int wmax = variant == kVarGemv ? 12 : 8;
        double best = 1e30;
        for (int kwc = 1; kwc <= kMaxWaves; kwc *= 2) {
            if (kwaves > 0 ? kwc != kwaves : (kwc != 1 && kwc != 4)) continue;
            const int smax = std::max(1, G / kwc);
            for (int sc = 1; sc <= smax; ++sc) {
                if (splits > 0 && sc != splits) continue;
                const long wgs = (long)(kwc == 1 ? ceil_div(NC, kWaves) : NC) * sc;
                const long waves = wgs * (kwc == 1 ? kWaves : kwc);
                const double rounds = std::ceil((double)waves / (256.0 * wmax));
                const double active = (double)std::min<long>(256, wgs);
                const double bw = std::min(5.8e6, active * 3.0e4);  // bytes per us
                double t = bytes / bw + 3.0 + (rounds - 1.0) * 3.0;
                if (sc > 1) t += 3.5 + sc * red_bytes / 5e6;
                if (t < best - 1e-9) {
                    best = t;
                    kw = kwc;
                    S = sc;
                }
            }
        }
        if (splits > 0) S = splits;
        if (kwaves > 0) kw = kwaves;
    } else {
        // LDS kernel (M > 16, or M = 15, 16 on wide linears): time model
        // calibrated on MI355X sweeps of forced split counts and workgroup
        // widths (WV = 4 or 8 chunks, one wave each),
        //   t(S, WV) = R(workgroups) * (G/S + 4) * t_group
        //            + [S > 1] * (2 us + S * M * NCpad * 8 bytes / 5 TB/s):
        // a CU holds two 4-wave workgroups side by side, and a CU running two
        // takes ~1.4x as long as one running one (down at M = 64: S = 16,
        // 512 workgroups, 53 us against 57 us for S = 8, 256 workgroups), so
        // for WV = 4, R = 1 up to 256 workgroups, else 1.4 per started round
        // of 512; an 8-wave workgroup fills a CU alone (two waves per SIMD)
        // and shares one activation copy between twice the chunks, R = 1.3
        // per round of 256 (gate at M = 64: 53.6 us against 58.6 us; q and k,
        // with few chunks, stay faster at WV = 4); every workgroup pays
        // start-up worth ~4 groups; t_group ~0.375 us per row block of 16;
        // S <= G/4: at least four groups per workgroup, below which start-up
        // and the partial traffic win over the model (k at M = 64: S = 16
        // 15.8 us, S = 22 16.7 us; at M = 32 12.2 against 13.7 us).  The least
        // t wins, ties to the smaller S and WV; a forced split count keeps S
        // and still chooses WV.
        //
        // Row slices: where even the most splits leave at least half the CUs
        // without a workgroup (k and v: 16 chunks, 64 workgroups at S = 16),
        // the row blocks are shared out between up to four workgroups per
        // column tile and split, each copying and multiplying only its own
        // rows (the weights are read once per slice, the later reads from
        // L2 or the MALL).  k at M = 64: 15.8 us in one slice, 12.3 in two,
        // 10.7 in four; at M = 32 12.2 against 10.1 in two.  Wider linears
        // lose (q at M = 64 equal in two, gate and down 5-20 % slower).
        const double red_bytes = (double)M * NC * kChunkN * 8;
        const int smax = std::max(1, G / 4);
        const long wgs_one = (long)ceil_div(NC, kWaves) * (splits > 0 ? splits : smax);
        int rs_cap = 1;
        while (rs_cap < 4 && rs_cap < mb && wgs_one * rs_cap * 2 <= 256) rs_cap *= 2;
        const int mbw = ceil_div(mb, rs_cap);
        rs = ceil_div(mb, mbw);
        double best = 1e30;
        int bs = 1;
        const double t_group = 0.375 * mbw;
        for (int wv = kWaves; wv <= kMaxWaves; wv *= 2) {
            const int ntiles = ceil_div(NC, wv);
            for (int s = 1; s <= smax || (splits > 0 && s <= splits); ++s) {
                if (splits > 0 && s != splits) continue;
                const double wgs = (double)ntiles * s * rs;
                const double rounds = wv == kWaves ? (wgs <= 256.0 ? 1.0 : 1.4 * std::ceil(wgs / 512.0))
                                                   : 1.3 * std::ceil(wgs / 256.0);
                double t = rounds * ((double)G / s + 4.0) * t_group;
                if (s > 1) t += 2.0 + s * red_bytes / 5e6;
                if (t < best - 1e-9) {
                    best = t;
                    bs = s;
                    lds_wv = wv;
                }
            }
        }
        S = bs;
    }
    S = std::max(1, std::min(S, G));
    int gps = ceil_div(G, S);
    S = ceil_div(G, gps);
    // the split-K workspace must hold S partial [M][NC*64] tiles
    while (S > 1 && (size_t)S * M * NC * kChunkN * 4 > ws_bytes) {
        ++gps;
        S = ceil_div(G, gps);
    }
    // every wave of a K-splitting workgroup needs a group of its own (the
    // last split holds the fewest groups)
    while (kw > 1 && G - (S - 1) * gps < kw) kw >>= 1;
    const int wg_chunks = variant == kVarLds ? lds_wv : kWaves;
    const int ntiles = kw == 1 ? ceil_div(NC, wg_chunks) : NC;
    p->kernel = kernel;
    p->variant = variant;
    p->mb = ceil_div(mb, rs);
    p->rs = rs;
    p->splits = S;
    p->kw = kw;
    p->gps = gps;
    p->ntiles = ntiles;
    p->grid = ntiles * S * rs;
    p->block = 64 * (kw == 1 ? wg_chunks : kw);
    p->lds = 0;
    if (variant == kVarLds) {
        p->lds = lds_ring_bytes(p->mb);
    }
    return 0;
}

hipError_t set_kernel_attributes() {
    // the LDS ring of the wide kernel stays under 64 KB; nothing to raise
    return hipSuccess;
}


static int grid_for(size_t total, int block) {
    size_t g = (total + block - 1) / block;
    if (g > 65535 * 4) g = 65535 * 4;
    return (int)std::max<size_t>(g, 1);
}

// Launch through hipLaunchKernel so the status returned is this launch's own
// (hipGetLastError could report an earlier, unrelated failure).
template <typename... Args>
static hipError_t launch(void (*kernel)(Args...), dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                         Args... args) {
    void* argv[] = {(void*)&args...};
    return hipLaunchKernel((const void*)kernel, grid, block, argv, lds, stream);
}

hipError_t launch_repack(const int32_t* qweight, const uint16_t* scales, const int32_t* zeros, int N, int K,
                         uint32_t* qweight_t, uint16_t* scales_t, uint16_t* zeros_t, hipStream_t stream) {
    const size_t NC = (size_t)ceil_div(N, kChunkN);
    const size_t words = NC * (K / kKBlock) * 256;
    hipError_t e = launch(repack_qweight_kernel, dim3(grid_for(words, 256)), dim3(256), 0, stream, qweight, N, K,
                          qweight_t, words);
    if (e != hipSuccess) return e;
    const size_t sz = NC * (K / kGroup) * 16;
    return launch(repack_scales_kernel, dim3(grid_for(sz, 256)), dim3(256), 0, stream, qweight, scales, zeros, N, K,
                  scales_t, zeros_t, sz);
}

hipError_t launch_unpack(const uint32_t* qweight_t, const uint16_t* zeros_t, int N, int K, uint8_t* q_out,
                         uint8_t* z_out, hipStream_t stream) {
    const size_t NC = (size_t)ceil_div(N, kChunkN);
    const size_t words = NC * (K / kKBlock) * 256;
    hipError_t e = launch(unpack_qweight_kernel, dim3(grid_for(words, 256)), dim3(256), 0, stream, qweight_t, N, K,
                          q_out, words, kNibbleMask, kBiasMagic);
    if (e != hipSuccess) return e;
    const size_t sz = NC * (K / kGroup) * 16;
    return launch(unpack_zeros_kernel, dim3(grid_for(sz, 256)), dim3(256), 0, stream, zeros_t, N, K, z_out, sz);
}

hipError_t launch_linear(const Plan& p, const uint16_t* x, const uint32_t* qweight_t, const uint16_t* scales_t,
                         const uint16_t* zeros_t, int M, int N, int K, void* y, int out_bf16, const Workspace& ws,
                         hipStream_t stream) {
    return launch_linear_io(p, x, K, qweight_t, scales_t, zeros_t, M, N, K, out_bf16 ? nullptr : (float*)y,
                            out_bf16 ? (uint16_t*)y : nullptr, 1.0f, ws, stream);
}

hipError_t launch_linear_io(const Plan& p, const uint16_t* x, int ldx, const uint32_t* qweight_t,
                            const uint16_t* scales_t, const uint16_t* zeros_t, int M, int N, int K, float* y,
                            uint16_t* yb, float alpha, const Workspace& ws, hipStream_t stream) {
    LinearArgs a;
    a.x = x;
    a.qt = (const u32x4*)qweight_t;
    a.st = (const uint2*)scales_t;
    a.zt = zeros_t;
    a.y = y;
    a.yb = yb;
    a.alpha = alpha;
    a.ws = ws.partial;
    a.M = M;
    a.N = N;
    a.K = K;
    a.ldx = ldx;
    a.NC = ceil_div(N, kChunkN);
    a.KB = K / kKBlock;
    a.G = K / kGroup;
    a.gps = p.gps;
    a.splits = p.splits;
    a.ntiles = p.ntiles;
    a.kw = p.kw;
    a.rs = p.rs;
    a.mask = kNibbleMask;
    a.magic = kBiasMagic;
    const dim3 grid(p.grid), block(p.block);
    hipError_t e;
    switch (p.variant) {
        case kVarGemv: e = launch(w4a16_gemv_kernel<kRingGemv>, grid, block, 0, stream, a); break;
        case kVarDirect: e = launch(w4a16_mfma_direct_kernel<1, kRingDirect1>, grid, block, 0, stream, a); break;
        default:
            if (p.block == 64 * kMaxWaves) {
                if (p.mb == 1)
                    e = launch(w4a16_mfma_lds_kernel<1, kMaxWaves>, grid, block, p.lds, stream, a);
                else if (p.mb == 2)
                    e = launch(w4a16_mfma_lds_kernel<2, kMaxWaves>, grid, block, p.lds, stream, a);
                else if (p.mb == 3)
                    e = launch(w4a16_mfma_lds_kernel<3, kMaxWaves>, grid, block, p.lds, stream, a);
                else
                    e = launch(w4a16_mfma_lds_kernel<4, kMaxWaves>, grid, block, p.lds, stream, a);
            } else if (p.mb == 1) {
                e = launch(w4a16_mfma_lds_kernel<1, kWaves>, grid, block, p.lds, stream, a);
            } else if (p.mb == 2) {
                e = launch(w4a16_mfma_lds_kernel<2, kWaves>, grid, block, p.lds, stream, a);
            } else if (p.mb == 3) {
                e = launch(w4a16_mfma_lds_kernel<3, kWaves>, grid, block, p.lds, stream, a);
            } else {
                e = launch(w4a16_mfma_lds_kernel<4, kWaves>, grid, block, p.lds, stream, a);
            }
    }
    if (e != hipSuccess || p.splits == 1) return e;
    const size_t total = (size_t)M * (N / 4);
    const dim3 rgrid(grid_for(total, 256)), rblock(256);
    const float* part = ws.partial;
    const int npad = a.NC * kChunkN;
    if (p.splits <= 2) return launch(splitk_reduce_kernel<2>, rgrid, rblock, 0, stream, part, a.y, a.yb, a.alpha, M, N, npad, p.splits);
    if (p.splits <= 4) return launch(splitk_reduce_kernel<4>, rgrid, rblock, 0, stream, part, a.y, a.yb, a.alpha, M, N, npad, p.splits);
    if (p.splits <= 8) return launch(splitk_reduce_kernel<8>, rgrid, rblock, 0, stream, part, a.y, a.yb, a.alpha, M, N, npad, p.splits);
    if (p.splits <= 16) return launch(splitk_reduce_kernel<16>, rgrid, rblock, 0, stream, part, a.y, a.yb, a.alpha, M, N, npad, p.splits);
    return launch(splitk_reduce_kernel<32>, rgrid, rblock, 0, stream, part, a.y, a.yb, a.alpha, M, N, npad, p.splits);
}

hipError_t launch_zero(float* y, size_t n, hipStream_t stream) {
    return launch(zero_kernel, dim3(grid_for(n, 256)), dim3(256), 0, stream, y, n);
}

hipError_t launch_bench_read(const void* buf, size_t bytes, uint32_t* sink, int blocks, hipStream_t stream) {
    // Measured on MI355X (graph-replayed, rotating past the MALL): up to
    // 64 MB, `blocks` (2048) workgroups with 4 loads per lane in flight
    // stream best; above, a quarter of them with 8.
    const size_t n16 = bytes / 16;
    const size_t nblk = n16 / 64;
    const bool big = bytes > (size_t(64) << 20);
    const int grid = (int)std::max<size_t>(1, std::min<size_t>(big ? blocks / 4 : blocks, std::max<size_t>(nblk, 1)));
    const size_t per = (nblk + grid - 1) / grid;
    if (big) return launch(bench_read_kernel<8>, dim3(grid), dim3(256), 0, stream, (const u32x4*)buf, n16, per, sink);
    return launch(bench_read_kernel<4>, dim3(grid), dim3(256), 0, stream, (const u32x4*)buf, n16, per, sink);
}

hipError_t launch_bench_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
    const size_t n16 = bytes / 16;
    return launch(bench_copy_kernel, dim3(grid_for(n16, 256)), dim3(256), 0, stream, (u32x4*)dst, (const u32x4*)src,
                  n16);
}

}  // namespace w4
