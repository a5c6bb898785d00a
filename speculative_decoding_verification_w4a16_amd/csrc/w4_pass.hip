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
// unit; that unit's activations are loaded once its producers are seen
// complete.  At the end of a unit each wave leaves its partial [rows x 64]
// sums in LDS and the waves meet at a barrier; one wave (rotating) then sums
// the partials in wave order, scales by the linear's alpha and stores the
// tile (fp32 and/or bf16) with agent-scope stores, which reach the device
// coherence point directly.
//
// Ordering without stalls: a wave polls the producer counters of its next
// unit at the start of the current unit's last round, before that round's
// reloads, so the answer is back by the unit's end without draining the
// ring.  The writing wave stores the tile before it loads the next unit's
// activations; as loads and stores retire in issue order, the wait for the
// first of those activations also covers the stores, and right after it the
// wave counts the unit done.  Where the next unit's producers are not yet
// done, the writing wave first drains its stores and counts its unit done,
// then every wave polls until they are -- a wave never waits with a unit of
// its own still uncounted.
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

// The table of linears is a separate `const __restrict__` kernel argument:
// read-only for the whole launch, so the compiler reads it with scalar loads,
// which wait on their own counter and never on the weight ring.
struct PassArgs {
    int n;                // linears
    int U;                // units (sum of the linears' chunk counts)
    int M;                // rows (verified tokens)
    uint32_t* done;       // [n] units done per linear (zero between launches)
    uint32_t* state;      // [0] workgroups exited, [1] error flag (sticky)
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

// One wave's share of a unit: groups [g0, g0 + ng) of chunk c of linear l,
// in at least two rounds of R steps (steps past ng are padding: their loads
// are clamped to the share's last group, their results unused).  Two rounds
// at least, so that every unit runs one first round and one last round.
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
    const int c = u - L.unit0;
    const int G = L.G, kw = L.kw;
    int g0 = 0, ng = 0;
    if (wave < kw) {
        g0 = G * wave / kw;
        ng = G * (wave + 1) / kw - g0;
    }
    WaveUnit w;
    w.ng = ng;
    w.nr = max(2, (ng + R - 1) / R);
    const int o = lane >> 4, t = lane & 15;
    w.wp = as_global((const u32x4*)L.qt) + ((size_t)c * (4 * G) + (size_t)g0 * 4) * 64 + lane;
    w.sp = as_global((const uint64_t*)L.st) + ((size_t)c * G + g0) * 16 + t;
    w.zp = as_global((const uint32_t*)L.zt) + ((size_t)c * G + g0) * 8 + (t >> 1);
    const int row = min(t, a.M - 1);  // the GEMV reads row 0 (M = 1)
    w.xp = as_global((const u32x4*)(L.x + (size_t)row * L.K + (size_t)g0 * kGroup + 8 * o));
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
        const bool xvalid = MB == 0 || t < a.M;
        const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{kOnesBf16x2, kOnesBf16x2, kOnesBf16x2, kOnesBf16x2});

        // producer counters of linear l, and the blocking wait for them; past
        // the limit the error flag is raised and the wait abandoned (the
        // results are then invalid, but every wave still exits)
        // (always kPassMaxDeps loads -- unused entries read counter 0 -- so
        // that the compiler counts the loads in flight exactly)
        auto poll = [&](int l, uint32_t (&pv)[kPassMaxDeps]) {
            const PassLinear& L = tab[l];
#pragma unroll
            for (int j = 0; j < kPassMaxDeps; ++j) pv[j] = load_agent(a.done + (j < L.ndep ? L.dep[j] : 0));
        };
        auto deps_ok = [&](int l, const uint32_t (&pv)[kPassMaxDeps]) {
            const PassLinear& L = tab[l];
            bool ok = true;
#pragma unroll
            for (int j = 0; j < kPassMaxDeps; ++j) ok = ok && (j >= L.ndep || pv[j] >= (uint32_t)L.dep_units[j]);
            return ok;
        };
        auto wait_deps = [&](int l) {
            const PassLinear& L = tab[l];
            for (int j = 0; j < L.ndep; ++j) {
                const uint32_t* cnt = a.done + L.dep[j];
                const uint32_t target = (uint32_t)L.dep_units[j];
                for (uint32_t it = 0;; ++it) {
                    if (load_agent(cnt) >= target) break;
                    if (it >= a.spin_limit || ((it & 63) == 63 && load_agent(a.state + 1) != 0u)) {
                        store_agent(a.state + 1, 1u);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                }
            }
        };

        int l = find_linear(tab, a, 0, u);
        WaveUnit cur = wave_unit<R>(tab, a, l, u, wave, lane, W);
        int un = u + G, ln = l;
        WaveUnit nxt = cur;
        if (un < a.U) {
            ln = find_linear(tab, a, l, un);
            nxt = wave_unit<R>(tab, a, ln, un, wave, lane, W);
        }
        uint32_t pv[kPassMaxDeps] = {0u, 0u, 0u, 0u};

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
                    const u32x4 raw = xvalid ? rx[d][kk] : u32x4{0, 0, 0, 0};
                    const bf16x8 av = __builtin_bit_cast(bf16x8, raw);
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
        int pend_l = -1;
        auto count_done = [&]() {
            if (pend_l >= 0 && lane == 0)
                __hip_atomic_fetch_add(a.done + pend_l, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            pend_l = -1;
        };

        // Rounds of R steps of the current share.  round_mid reloads each slot
        // with the share's own step R ahead (weights, then activations);
        // round_last polls the next unit's producers, then reloads each slot
        // with the next unit's first R groups of weights only.  The first
        // round of a unit (which also counts the previous unit done once its
        // stores have retired), the middle rounds (a loop) and the last are
        // separate code, so every loop header sees one pattern of loads in
        // flight and the compiler's wait counts stay exact (a separate copy
        // for one-round units doubled the live registers: units have two
        // rounds at least).
        auto round_first = [&]() {
#pragma unroll
            for (int d = 0; d < R; ++d) {
                if (d < cur.ng) step(d);
                if (d == 0) count_done();  // step 0 waited for loads issued after the stores
                load_w(d, cur, d + R);
                load_x(d, cur, d + R);
            }
        };
        auto round_mid = [&](int r0) {
#pragma unroll
            for (int d = 0; d < R; ++d) {
                const int i = r0 * R + d;
                if (i < cur.ng) step(d);
                load_w(d, cur, i + R);
                load_x(d, cur, i + R);
            }
        };
        auto round_last = [&](int r0) {
            poll(ln, pv);
#pragma unroll
            for (int d = 0; d < R; ++d) {
                const int i = r0 * R + d;
                if (i < cur.ng) step(d);
                load_w(d, nxt, d);
            }
        };

        // the first unit: its weights now, its activations once its producers are done
#pragma unroll
        for (int d = 0; d < R; ++d) load_w(d, cur, d);
        wait_deps(l);
        for (int cnt = 0;; ++cnt) {
#pragma unroll
            for (int d = 0; d < R; ++d) load_x(d, cur, d);
            // issue all four in slot order here: the compiler would otherwise
            // sink slot 0's loads into the step that uses them, behind the
            // others, and the first wait would then drain the whole ring
            asm volatile("" ::: "memory");
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                yg[j] = 0.0f;
                ym[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            }
            round_first();
            for (int r0 = 1; r0 < cur.nr - 1; ++r0) round_mid(r0);
            round_last(cur.nr - 1);
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
            if (wave == cnt % W) {
                // this wave writes the tile: W partials summed in wave order
                const PassLinear& L = tab[l];
                const int c = u - L.unit0;
                const float alpha = L.alpha;
                const int buf = cnt & 1;
                if (MB == 0) {
                    float v = 0.0f;
                    for (int w = 0; w < W; ++w) v += part[buf][w][lane];
                    const int n = c * kChunkN + lane;
                    const float y0 = v * alpha;
                    if (L.y && n < L.N) store_agent((uint32_t*)(L.y + n), __float_as_uint(y0));
                    if (L.yb) {
                        const uint32_t b = f32_to_bf16_rne(y0);
                        const uint32_t b1 = (uint32_t)__shfl_down((int)b, 1);
                        if ((lane & 1) == 0 && n < L.N) store_agent((uint32_t*)(L.yb + n), b | (b1 << 16));
                    }
                } else {
                    const int r = lane >> 2, cb = (lane & 3) * 16;  // row r, 16 columns from cb
                    float v[16];
#pragma unroll
                    for (int i = 0; i < 16; ++i) v[i] = 0.0f;
                    for (int w = 0; w < W; ++w)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const f32x4 p4 = *(const f32x4*)&part[buf][w][r * kChunkN + cb + 4 * q];
                            v[4 * q + 0] += p4[0];
                            v[4 * q + 1] += p4[1];
                            v[4 * q + 2] += p4[2];
                            v[4 * q + 3] += p4[3];
                        }
                    if (r < a.M) {
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int n = c * kChunkN + cb + 4 * q;
                            if (n >= L.N) continue;  // N % 8 == 0: a quad is all in or all out
                            const float y0 = v[4 * q] * alpha, y1 = v[4 * q + 1] * alpha;
                            const float y2 = v[4 * q + 2] * alpha, y3 = v[4 * q + 3] * alpha;
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
                    }
                }
                pend_l = l;
            }
            if (un >= a.U) break;
            if (!deps_ok(ln, pv)) {
                // producers still running: count this wave's own unit first
                if (pend_l >= 0) {
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                    count_done();
                }
                wait_deps(ln);
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
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (wave == 0) {
        uint32_t old = 0;
        if (lane == 0) old = __hip_atomic_fetch_add(a.state, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        old = (uint32_t)__shfl((int)old, 0);
        if (old == (uint32_t)G - 1) {
            for (int i = lane; i < a.n; i += 64) store_agent(a.done + i, 0u);
            if (lane == 0) store_agent(a.state, 0u);
        }
    }
}

}  // namespace

hipError_t launch_pass(const PassLinear* tab, int n, int U, int M, uint32_t* done, uint32_t* state,
                       uint32_t spin_limit, int grid, hipStream_t stream) {
    PassArgs a;
    a.n = n;
    a.U = U;
    a.M = M;
    a.done = done;
    a.state = state;
    a.spin_limit = spin_limit;
    a.mask = kNibbleMask;
    a.magic = kBiasMagic;
    void* argv[] = {(void*)&tab, (void*)&a};
    const dim3 block(64 * kPassWaves);
    if (M == 1)
        return hipLaunchKernel((const void*)w4_pass_kernel<0, kPassWaves, kPassRing>, dim3(grid), block, argv, 0,
                               stream);
    return hipLaunchKernel((const void*)w4_pass_kernel<1, kPassWaves, kPassRing>, dim3(grid), block, argv, 0,
                           stream);
}

hipError_t pass_occupancy(int M, int* per_cu) {
    const void* k = M == 1 ? (const void*)w4_pass_kernel<0, kPassWaves, kPassRing>
                           : (const void*)w4_pass_kernel<1, kPassWaves, kPassRing>;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, k, 64 * kPassWaves, 0);
}

}  // namespace w4
