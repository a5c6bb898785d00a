// A whole verify pass in one launch, for the plain-decode and sequence-draft
// sizes (M <= 16).
//
// The pages' target model verifies a draft with one forward pass that runs
// every drafted token through every 4-bit linear ("Speculative Decoding
// Meets Quantization", Abstract; ordoresearch.ai review, "Research
// Landscape"), and at these M that pass is bound by reading the packed
// weights ("memory bandwidth -- often the primary bottleneck").  Launching
// each linear on its own leaves the memory system idle between launches: a
// launch has to drain before the next may start, and the next one's first
// loads then take a full memory round trip.  Over the 561 linears of a
// Llama-3-70B pass that costs about a third of the pass.
//
// This kernel keeps every CU streaming weights across linear boundaries.
// It is persistent: one workgroup of W waves per CU, each workgroup taking
// the pass's units (a unit is one 64-column chunk of one linear over its
// whole K) in pass order, round-robin (unit u goes to workgroup u mod grid).
// A linear may read the output of earlier linears (its producers, given per
// linear): its units multiply only after every unit of every producer has
// stored its output and counted itself done, but their weights -- which
// depend on no activation -- are loaded ahead, while the previous unit is
// still being computed.
//
// The W waves split a unit's K range (whole groups) and run the streaming
// kernels' inner loops (the VALU GEMV at M = 1, bf16 MFMA with the
// activation rows as A operands at M = 2..16) over a register ring of R
// groups of weights, scales, zeros and activations in flight per wave (all
// at one depth: loads retire in issue order, so waiting for a later load
// also waits for every older one).  The last round of R steps of a unit
// reloads the ring with the wave's first R groups of weights of its next
// unit; that unit's activations follow once its producers are complete.  At
// the end of a unit each wave leaves its partial [rows x 64] sums in LDS and
// the waves meet at a barrier; one wave (rotating) then sums the partials in
// wave order, scales by the linear's alpha and stores the tile (fp32 and/or
// bf16) with agent-scope stores, which reach the device coherence point
// directly.
//
// Completion counting: unit c of a linear counts on one of 64 sub-counters
// (c mod 64), each on its own 64-byte line -- atomics on one address are
// performed one at a time, and a single counter per linear would queue
// every unit's increment behind all the others.  A consumer's lane j reads
// sub-counter j; the producer is complete when every lane has seen its
// count.
//
// Ordering without stalls: within a linear, and across linears with the
// same producers, the producers are already known complete, so the last
// round loads the next unit's activations right away and the ring never
// drains.  The writing wave then counts its unit done at step 0 of the next
// unit's second round, once the loads issued after its tile stores have
// retired (in-order retirement covers the stores).  At a linear whose
// producers are not known complete, the writing wave retires its stores and
// counts its unit done at once (no wave waits with a unit of its own
// uncounted), wave 0 polls the producers' sub-counters, the workgroup meets
// at a barrier, and every wave loads the activations of its next unit (its
// weights are in the ring already).
//
// Units are numbered in pass order and a linear's producers come before it,
// so the lowest unit not yet done has all its producers done: with every
// workgroup resident (one per CU, the grid is at most the CU count) the pass
// always progresses.  Every wait is bounded: past `spin_limit` polls the
// wave raises the pass's error flag and goes on, so every wave exits.  The
// last workgroup to exit resets the counters for the next launch (no memset,
// so the launch can be captured in a HIP graph and replayed).
//
// Activations written by one workgroup and read by another are read with
// ordinary loads: each output buffer is written once per launch, before any
// consumer reads it (the producer counters order that), it shares no 128-byte
// line with any other buffer of the pass (checked on the host), and the
// caches hold no copy of it from before the launch (the kernel boundary
// invalidates them).
#include "w4_device.h"
#include "w4_internal.h"

namespace w4 {

namespace {

// Stores through pointers read from the table go to the global address space
// explicitly (a generic pointer would give flat stores, which count on both
// wait counters).
__device__ __forceinline__ void store_agent(uint32_t* p, uint32_t v) {
    __hip_atomic_store((__attribute__((address_space(1))) uint32_t*)p, v, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(uint64_t* p, uint64_t v) {
    __hip_atomic_store((__attribute__((address_space(1))) uint64_t*)p, v, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_agent(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_agent64(const uint64_t* p) {
    return __hip_atomic_load((const __attribute__((address_space(1))) uint64_t*)p, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}

// The table of linears is a separate `const __restrict__` kernel argument:
// read-only for the whole launch, so the compiler reads it with scalar loads,
// which wait on their own counter and never on the weight ring.
struct PassArgs {
    int n;                // linears
    int U;                // units (sum over the linears of chunks x K slices)
    int M;                // rows (verified tokens)
    uint32_t* done;       // chunks done per linear: kPassSub sub-counters each (zero between launches)
    uint32_t* arr;        // slices arrived per split chunk (zero between launches)
    int narr;
    uint32_t* state;      // [0] workgroups exited, [1] error flag (sticky)
    float* part;          // partial tiles of the K-split units
    uint32_t spin_limit;  // polls before a wait gives up
    uint32_t mask, magic; // the unpack's constants (see unpack_biased)
};

// The linear holding unit u, searching forward from linear l.
__device__ __forceinline__ int find_linear(const PassLinear* __restrict__ tab, const PassArgs& a, int l, int u) {
    while (l + 1 < a.n && tab[l + 1].unit0 <= u) ++l;
    return l;
}

// Pointers read from the table are generic to the compiler, which would load
// through them with flat instructions (counted on both wait counters, so
// every use would wait for all loads in flight); the wave's stream pointers
// are cast to the global address space instead.
#define W4_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ const W4_GLOBAL T* as_global(const T* p) {
    return (const W4_GLOBAL T*)p;
}

// A unit is slice s of chunk c of linear l (the linear's units in chunk
// order, its S slices of K adjacent): groups [s gps, min(G, (s + 1) gps)).
// One wave's share of it is groups [g0, g0 + ng), in at least two rounds of R
// steps (steps past ng are padding: their loads are clamped to the share's
// last group, their results unused).  Two rounds at least, so that every
// unit runs one first round and one last round.
struct WaveUnit {
    int ng, nr;
    const W4_GLOBAL u32x4* wp;     // weights of group g0, this lane's 16 bytes
    const W4_GLOBAL uint64_t* sp;  // scales of group g0, this lane's column quad
    const W4_GLOBAL uint32_t* zp;  // zeros of group g0: the aligned pair of records holding this lane's
    const W4_GLOBAL u32x4* xp;     // activations of group g0, this lane's octet (and row)
};

template <int R>
__device__ __forceinline__ WaveUnit wave_unit(const PassLinear* __restrict__ tab, const PassArgs& a, int l, int u,
                                              int wave, int lane, int W) {
    const PassLinear& L = tab[l];
    const int cs = u - L.unit0;
    const int c = cs / L.S;
    const int G = L.G, kw = L.kw;
    const int sg0 = (cs - c * L.S) * L.gps;
    const int sng = min(G, sg0 + L.gps) - sg0;
    int g0 = sg0, ng = 0;
    if (wave < kw) {
        g0 = sg0 + sng * wave / kw;
        ng = sg0 + sng * (wave + 1) / kw - g0;
    }
    WaveUnit w;
    w.ng = ng;
    w.nr = max(2, (ng + R - 1) / R);
    const int o = lane >> 4, t = lane & 15;
    w.wp = as_global((const u32x4*)L.qt) + ((size_t)c * (4 * G) + (size_t)g0 * 4) * 64 + lane;
    w.sp = as_global((const uint64_t*)L.st) + ((size_t)c * G + g0) * 16 + t;
    w.zp = as_global((const uint32_t*)L.zt) + ((size_t)c * G + g0) * 8 + (t >> 1);
    const int row = min(t, a.M - 1);  // the GEMV reads row 0 (M = 1)
    w.xp = as_global((const u32x4*)(L.x + (size_t)row * L.ldx + (size_t)g0 * kGroup + 8 * o));
    (void)W;
    return w;
}

// MB = 0: the VALU GEMV (M = 1); MB = 1: bf16 MFMA over one block of 16 rows.
template <int MB, int W, int R>
__global__ __launch_bounds__(64 * W) void w4_pass_kernel(const PassLinear* __restrict__ tab, PassArgs a) {
    static_assert(R == 4, "the round structure assumes four steps");
    constexpr int kRows = MB == 0 ? 1 : 16;
    __shared__ __align__(16) float part[2][W][kRows * kChunkN];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int G = gridDim.x;
    int u = blockIdx.x;

    if (u < a.U) {
        const int o = lane >> 4, t = lane & 15;
        const uint32_t mask = a.mask, magic = to_vgpr(a.magic);
        const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{kOnesBf16x2, kOnesBf16x2, kOnesBf16x2, kOnesBf16x2});

        // Completion of a producer: its chunk c counts on sub-counter c % 64,
        // so lane j reads sub-counter j and compares it with the number of
        // chunks that count there; the producer is complete when every lane
        // agrees.  One wave of the workgroup polls (wave 0); past the limit
        // it raises the error flag and gives up (the results are then
        // invalid, but every wave still exits).
        auto sub = [&](int l) { return a.done + ((size_t)l * kPassSub + lane) * kPassSubStride; };
        auto expected = [&](int nc) { return (uint32_t)(nc / kPassSub + (lane < nc % kPassSub ? 1 : 0)); };
        auto wait_deps = [&](int l) {
            const PassLinear& L = tab[l];
            if (L.ndep == 0) return;
            for (uint32_t it = 0;; ++it) {
                // every producer in one round trip
                uint32_t v[kPassMaxDeps];
#pragma unroll
                for (int j = 0; j < kPassMaxDeps; ++j) v[j] = j < L.ndep ? load_agent(sub(L.dep[j])) : 0u;
                bool ok = true;
#pragma unroll
                for (int j = 0; j < kPassMaxDeps; ++j) ok = ok && (j >= L.ndep || v[j] >= expected(L.dep_units[j]));
                if (__ballot(!ok) == 0ull) break;
                if (it >= a.spin_limit || ((it & 63) == 63 && load_agent(a.state + 1) != 0u)) {
                    if (lane == 0) store_agent(a.state + 1, 1u);
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        };
        // The producers of every linear with the dependency class `ok` (the
        // same set of producers) are known complete: its units need no wait.
        int ok = -1;
        auto known_ready = [&](int l) { return tab[l].ndep == 0 || tab[l].dep_class == ok; };

        int l = find_linear(tab, a, 0, u);
        WaveUnit cur = wave_unit<R>(tab, a, l, u, wave, lane, W);
        int un = u + G, ln = l;
        WaveUnit nxt = cur;
        if (un < a.U) {
            ln = find_linear(tab, a, l, un);
            nxt = wave_unit<R>(tab, a, ln, un, wave, lane, W);
        }

        u32x4 rw[R][4];
        uint2 rs[R];
        uint32_t rz[R];
        u32x4 rx[R][4];
        // weights, scales and zeros of step i of a share into ring slot d
        auto load_w = [&](int d, const WaveUnit& sh, int i) {
            __builtin_amdgcn_sched_barrier(0);  // keep the reload after the slot's last use
            const int g = min(i, max(sh.ng, 1) - 1);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) rw[d][kk] = __builtin_nontemporal_load(sh.wp + (g * 4 + kk) * 64);
            const uint64_t sv = __builtin_nontemporal_load(sh.sp + g * 16);
            rs[d] = make_uint2((uint32_t)sv, (uint32_t)(sv >> 32));
            rz[d] = __builtin_nontemporal_load(sh.zp + g * 8);
        };
        auto load_x = [&](int d, const WaveUnit& sh, int i) {
            const int g = min(i, max(sh.ng, 1) - 1);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) rx[d][kk] = sh.xp[g * 16 + kk * 4];
        };

        float yg[4];  // GEMV: this lane's 4 columns (one k octet of each)
        f32x4 ym[4];  // MFMA: rows 4o + r of the lane's column in each n-tile
        // one group: ring slot d.  A lane's zero record (16 bits) is half of
        // the 32-bit pair it loads: a 16-bit load would be widened with an
        // AND at the loop latch, which waits for the load just issued.
        const uint32_t zshift = 16u * (t & 1);
        auto step = [&](int d) {
            float sj[4];
            decode_scales(rs[d], sj);
            const uint32_t zw = rz[d] >> zshift;
            if (MB == 0) {
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
#pragma unroll
                for (int j = 0; j < 4; ++j) yg[j] = fmaf(sj[j], fmaf(-biased_zero(zw, j), xs, acc[j]), yg[j]);
            } else {
                f32x4 acc[4], accx;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    // rows past M hold row M - 1 again (their sums are never stored)
                    const bf16x8 av = __builtin_bit_cast(bf16x8, rx[d][kk]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const bf16x8 bv = __builtin_bit_cast(bf16x8, unpack_biased(rw[d][kk][j], mask, magic));
                        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            av, bv, kk == 0 ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : acc[j], 0, 0, 0);
                    }
                    accx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        av, ones, kk == 0 ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : accx, 0, 0, 0);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float cz = biased_zero(zw, j);
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) ym[j][rr] = fmaf(sj[j], fmaf(-cz, accx[rr], acc[j][rr]), ym[j][rr]);
                }
            }
        };

        // the unit this wave stored and has not counted yet (-1: none)
        int pend_l = -1, pend_c = 0;
        auto count_done = [&]() {
            if (pend_l >= 0 && lane == 0)
                __hip_atomic_fetch_add(a.done + ((size_t)pend_l * kPassSub + pend_c % kPassSub) * kPassSubStride, 1u,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            pend_l = -1;
        };
        // Loads a step issues: 4 of weights, 1 of scales, 1 of zeros, 4 of
        // activations.  At step 0 of the second round the whole first round's
        // loads were issued after the tile stores; waiting until no more than
        // that many are outstanding retires the stores (the step itself
        // usually waits longer already -- not when the step is padding).
        constexpr int kLoadsPerStep = 10;
        auto count_done_stored = [&]() {
            if (pend_l >= 0) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(R * kLoadsPerStep) : "memory");
            count_done();
        };
        // One round of R steps; each step reloads its slot R steps ahead
        // within the unit.
        auto round = [&](int r) {
#pragma unroll
            for (int d = 0; d < R; ++d) {
                const int i = r * R + d;
                if (i < cur.ng) step(d);
                if (r == 1 && d == 0) count_done_stored();
                load_w(d, cur, i + R);
                load_x(d, cur, i + R);
            }
        };
        // The last round reloads the ring with the next unit's weights; its
        // activations follow, for all R slots, once its producers are
        // complete: at once when they are known complete, else after the
        // wait.  Both ways the ring is loaded in the same order (weights of
        // slots 0..R-1, then activations of slots 0..R-1), so the compiler's
        // wait counts hold for either.
        // `hold`: this wave writes the tile and then waits for producers --
        // it reloads this unit's first group instead (recently read, so a
        // cache hit), leaving little in flight behind its tile stores, which
        // it retires before counting; it loads the next unit's weights after
        // the wait.
        auto last_round = [&](int r, bool hold) {
#pragma unroll
            for (int d = 0; d < R; ++d) {
                const int i = r * R + d;
                if (i < cur.ng) step(d);
                if (r == 1 && d == 0) count_done_stored();
                load_w(d, hold ? cur : nxt, hold ? 0 : d);
            }
        };
        auto load_next_x = [&]() {
#pragma unroll
            for (int d = 0; d < R; ++d) {
                __builtin_amdgcn_sched_barrier(0);  // in slot order
                load_x(d, nxt, d);
            }
        };

        // the first unit: its producers, then its first R groups
        if (wave == 0) wait_deps(l);
        __syncthreads();
        ok = tab[l].dep_class;
#pragma unroll
        for (int d = 0; d < R; ++d) load_w(d, cur, d);
#pragma unroll
        for (int d = 0; d < R; ++d) {
            __builtin_amdgcn_sched_barrier(0);
            load_x(d, cur, d);
        }
        for (int cnt = 0;; ++cnt) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                yg[j] = 0.0f;
                ym[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            }
            // round 0 apart: it starts from the ring as a unit start leaves it
            // (weights, then activations), the later rounds from a round's
            // order (slot by slot) -- each gets its own exact wait counts
            round(0);
            for (int r = 1; r < cur.nr - 1; ++r) round(r);
            const bool more = un < a.U;
            const bool fast = more && known_ready(ln);
            const bool writer = wave == cnt % W;  // the wave that stores this unit's tile
            last_round(cur.nr - 1, writer && !fast);
            if (fast) load_next_x();
            // this wave's partial sums of the unit, into LDS
            float* dst = part[cnt & 1][wave];
            if (MB == 0) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    yg[j] += __shfl_xor(yg[j], 16);
                    yg[j] += __shfl_xor(yg[j], 32);
                }
                if (o == 0)
#pragma unroll
                    for (int j = 0; j < 4; ++j) dst[16 * j + t] = yg[j];
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) dst[(4 * o + rr) * kChunkN + 16 * j + t] = ym[j][rr];
            }
            lds_barrier();  // the W partials of the unit are complete
            if (writer) {
                // This wave writes the tile: the W partials summed in wave
                // order, scaled by alpha, stored as fp32 and/or bf16.  A K
                // slice of a split chunk stores its unscaled partial tile
                // instead; the chunk's last slice to arrive sums the S
                // partial tiles in slice order and stores the chunk's tile.
                const PassLinear& L = tab[l];
                const int cs = u - L.unit0;
                const int c = cs / L.S;
                const int buf = cnt & 1;
                constexpr int kTile = kRows * kChunkN;
                // the lane's element(s) of the tile: GEMV column `lane`;
                // MFMA row r, columns cb + 4q .. + 3
                const int r = lane >> 2, cb = (lane & 3) * 16;
                auto wave_sum = [&](int q) {
                    if (MB == 0) {
                        float v = 0.0f;
                        for (int w = 0; w < W; ++w) v += part[buf][w][lane];
                        return f32x4{v, 0.0f, 0.0f, 0.0f};
                    }
                    f32x4 v = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                    for (int w = 0; w < W; ++w) v += *(const f32x4*)&part[buf][w][r * kChunkN + cb + 4 * q];
                    return v;
                };
                auto store_tile = [&](auto&& value) {
                    const float alpha = L.alpha;
                    if (MB == 0) {
                        const float y0 = value(0)[0] * alpha;
                        const int n = c * kChunkN + lane;
                        if (L.y && n < L.N) store_agent((uint32_t*)(L.y + n), __float_as_uint(y0));
                        if (L.yb) {
                            const uint32_t b = f32_to_bf16_rne(y0);
                            const uint32_t b1 = (uint32_t)__shfl_down((int)b, 1);
                            if ((lane & 1) == 0 && n < L.N) store_agent((uint32_t*)(L.yb + n), b | (b1 << 16));
                        }
                        return;
                    }
                    // one quad at a time (the next unit's ring is in flight:
                    // few registers to spare)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int n = c * kChunkN + cb + 4 * q;
                        // N % 8 == 0: a quad is all in or all out
                        if (r >= a.M || n >= L.N) continue;
                        const f32x4 v = value(q);
                        const float y0 = v[0] * alpha, y1 = v[1] * alpha;
                        const float y2 = v[2] * alpha, y3 = v[3] * alpha;
                        const size_t off = (size_t)r * L.N + n;
                        if (L.y) {
                            store_agent((uint64_t*)(L.y + off),
                                        (uint64_t)__float_as_uint(y0) | ((uint64_t)__float_as_uint(y1) << 32));
                            store_agent((uint64_t*)(L.y + off + 2),
                                        (uint64_t)__float_as_uint(y2) | ((uint64_t)__float_as_uint(y3) << 32));
                        }
                        if (L.yb) {
                            const uint64_t lo = f32_to_bf16_rne(y0) | ((uint32_t)f32_to_bf16_rne(y1) << 16);
                            const uint64_t hi = f32_to_bf16_rne(y2) | ((uint32_t)f32_to_bf16_rne(y3) << 16);
                            store_agent((uint64_t*)(L.yb + off), lo | (hi << 32));
                        }
                    }
                };
                if (L.S == 1) {
                    store_tile(wave_sum);
                    pend_l = l;
                    pend_c = c;
                } else {
                    float* tile = a.part + (size_t)(L.part0 + cs) * kTile;
                    if (MB == 0) {
                        store_agent((uint32_t*)(tile + lane), __float_as_uint(wave_sum(0)[0]));
                    } else {
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            if (r >= a.M) continue;
                            const f32x4 v = wave_sum(q);
                            float* p4 = tile + r * kChunkN + cb + 4 * q;
                            store_agent((uint64_t*)p4, (uint64_t)__float_as_uint(v[0]) |
                                                           ((uint64_t)__float_as_uint(v[1]) << 32));
                            store_agent((uint64_t*)(p4 + 2), (uint64_t)__float_as_uint(v[2]) |
                                                                 ((uint64_t)__float_as_uint(v[3]) << 32));
                        }
                    }
                    // the partial tile retires before the slice arrives
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                    uint32_t old = 0;
                    if (lane == 0)
                        old = __hip_atomic_fetch_add(a.arr + L.arr0 + c, 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
                    old = (uint32_t)__builtin_amdgcn_readfirstlane((int)__shfl((int)old, 0));
                    if (old == (uint32_t)L.S - 1) {
                        // every other slice stored its tile before arriving
                        const float* t0 = a.part + (size_t)(L.part0 + c * L.S) * kTile;
                        store_tile([&](int q) {
                            f32x4 v = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                            for (int s2 = 0; s2 < L.S; ++s2) {
                                const float* p4 = t0 + (size_t)s2 * kTile;
                                if (MB == 0) {
                                    v[0] += __uint_as_float(load_agent((const uint32_t*)(p4 + lane)));
                                } else {
                                    const uint64_t lo = load_agent64((const uint64_t*)(p4 + r * kChunkN + cb + 4 * q));
                                    const uint64_t hi =
                                        load_agent64((const uint64_t*)(p4 + r * kChunkN + cb + 4 * q + 2));
                                    v[0] += __uint_as_float((uint32_t)lo);
                                    v[1] += __uint_as_float((uint32_t)(lo >> 32));
                                    v[2] += __uint_as_float((uint32_t)hi);
                                    v[3] += __uint_as_float((uint32_t)(hi >> 32));
                                }
                            }
                            return v;
                        });
                        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                        pend_l = l;
                        pend_c = c;
                        count_done();
                    }
                }
            }
            if (!more) break;
            if (!fast) {
                // The next unit's producers are not known complete.  The
                // writer retires its stores and counts its unit done (no
                // wave waits with a unit of its own uncounted); wave 0 waits
                // for the producers; then every wave loads the next unit's
                // activations (their weights are in the ring already, except
                // the writer's).
                if (writer) {
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                    count_done();
                }
                if (wave == 0) wait_deps(ln);
                __syncthreads();
                ok = tab[ln].dep_class;
                if (writer)
#pragma unroll
                    for (int d = 0; d < R; ++d) load_w(d, nxt, d);
                load_next_x();
            }
            u = un;
            l = ln;
            cur = nxt;
            un = u + G;
            if (un < a.U) {
                ln = find_linear(tab, a, l, un);
                nxt = wave_unit<R>(tab, a, ln, un, wave, lane, W);
            }
        }
        // the last unit's tile: its stores retire, then it counts
        if (pend_l >= 0) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            count_done();
        }
    }

    // exit: the last workgroup out resets the counters for the next launch
    __shared__ uint32_t last;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0)
        last = __hip_atomic_fetch_add(a.state, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)G - 1;
    __syncthreads();
    if (last) {
        const size_t subs = (size_t)a.n * kPassSub;
        for (size_t i = threadIdx.x; i < subs; i += blockDim.x) store_agent(a.done + i * kPassSubStride, 0u);
        for (int i = threadIdx.x; i < a.narr; i += blockDim.x) store_agent(a.arr + i, 0u);
        if (threadIdx.x == 0) store_agent(a.state, 0u);
    }
}

}  // namespace

hipError_t launch_pass(const PassLaunch& l, hipStream_t stream) {
    PassArgs a;
    a.n = l.n;
    a.U = l.U;
    a.M = l.M;
    a.done = l.done;
    a.arr = l.done + (size_t)l.n * kPassSub * kPassSubStride;
    a.narr = l.arrivals;
    a.state = l.state;
    a.part = l.part;
    a.spin_limit = l.spin_limit;
    a.mask = kNibbleMask;
    a.magic = kBiasMagic;
    const PassLinear* tab = l.tab;
    void* argv[] = {(void*)&tab, (void*)&a};
    const dim3 block(64 * kPassWaves);
    if (l.M == 1)
        return hipLaunchKernel((const void*)w4_pass_kernel<0, kPassWaves, kPassRing>, dim3(l.grid), block, argv, 0,
                               stream);
    return hipLaunchKernel((const void*)w4_pass_kernel<1, kPassWaves, kPassRing>, dim3(l.grid), block, argv, 0,
                           stream);
}

hipError_t pass_occupancy(int M, int* per_cu) {
    const void* k = M == 1 ? (const void*)w4_pass_kernel<0, kPassWaves, kPassRing>
                           : (const void*)w4_pass_kernel<1, kPassWaves, kPassRing>;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, k, 64 * kPassWaves, 0);
}

}  // namespace w4
