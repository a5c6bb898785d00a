// Internal interface between the C ABI (w4a16_api.cpp) and the kernels
// (w4a16_kernels.hip).  Not installed; the public ABI is include/w4a16.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/w4a16.h"

namespace w4 {

constexpr int kChunkN = 64;   // output columns per chunk (4 MFMA n-tiles of 16)
constexpr int kKBlock = 32;   // k per MFMA k-block (one 16x16x32 bf16 MFMA)
constexpr int kGroup = 128;   // quantisation group along k
constexpr int kWaves = 4;     // waves per workgroup (one chunk each)
constexpr int kThreads = kWaves * 64;
constexpr int kMaxWaves = 8;              // waves per workgroup when they split one chunk's K range
constexpr int kMaxThreads = kMaxWaves * 64;

enum KernelId { kAuto = 0, kGemv = 1, kMfma = 2 };

// Kernel variants behind the ids: the VALU GEMV (M = 1), the MFMA kernel
// with A operands loaded straight from global memory (M <= 16), and the MFMA
// kernel with activations copied into an LDS ring (M = 17..64, and M = 15, 16
// on linears of 4096 or more columns).
enum Variant { kVarGemv = 0, kVarDirect = 1, kVarLds = 2 };

struct Plan {
    int kernel;   // kGemv or kMfma
    int variant;  // Variant
    int mb;       // m-blocks of 16 rows (MFMA) per workgroup
    int rs;       // row slices: workgroups per column tile and split along M (LDS kernel), mb blocks each
    int splits;   // K splits (workgroups per column tile)
    int kw;       // waves per workgroup splitting one chunk's K range (1: one chunk per wave)
    int gps;      // groups per split
    int ntiles;   // column tiles (one workgroup's chunks each)
    int grid;     // workgroups
    int block;    // threads per workgroup
    int lds;      // dynamic LDS bytes per workgroup
};

struct Workspace {
    float* partial;  // split-K partial sums, [S][M][NC*64] fp32
    size_t partial_bytes;
};

// LDS budget per workgroup for the staged activation tile.
constexpr int kLdsLimit = 160 * 1024 - 256;  // room for the small static LDS

// Split-K workspace size (per device).
constexpr size_t kWorkspaceBytes = size_t(64) << 20;

// The allocation-free entry point's static split-K scratch (per device, the
// same size as the workspace, so both plan every call alike).
constexpr size_t kNoAllocScratchBytes = kWorkspaceBytes;
static_assert(kNoAllocScratchBytes == W4_NOALLOC_SCRATCH_BYTES, "the header states the scratch size");

// Device address of the current device's static scratch (looked up once per
// device with hipGetSymbolAddress; no allocation).
hipError_t noalloc_scratch(Workspace* ws);

// kwaves: 0 = the planner's choice, else 1, 2, 4 or 8 (M <= 16 only; the
// M > 16 kernel always uses 1).  Returns non-zero for an impossible request.
int plan_linear(int M, int N, int K, int kernel, int splits, int kwaves, size_t ws_bytes, Plan* p);

hipError_t set_kernel_attributes();

hipError_t launch_repack(const int32_t* qweight, const uint16_t* scales, const int32_t* zeros, int N, int K,
                         uint32_t* qweight_t, uint16_t* scales_t, uint16_t* zeros_t, hipStream_t stream);

hipError_t launch_unpack(const uint32_t* qweight_t, const uint16_t* zeros_t, int N, int K, uint8_t* q_out,
                         uint8_t* z_out, hipStream_t stream);

// y: fp32 [M][N], or bf16 bits [M][N] when out_bf16.
hipError_t launch_linear(const Plan& p, const uint16_t* x, const uint32_t* qweight_t, const uint16_t* scales_t,
                         const uint16_t* zeros_t, int M, int N, int K, void* y, int out_bf16, const Workspace& ws,
                         hipStream_t stream);

// The same with both outputs optional (fp32 y and/or bf16 yb, at least one)
// and the result scaled by alpha.
hipError_t launch_linear_io(const Plan& p, const uint16_t* x, int ldx, const uint32_t* qweight_t,
                            const uint16_t* scales_t, const uint16_t* zeros_t, int M, int N, int K, float* y,
                            uint16_t* yb, float alpha, const Workspace& ws, hipStream_t stream);

hipError_t launch_zero(float* y, size_t n, hipStream_t stream);

// ---------------------------------------------------------------------------
// the verify pass in one launch (w4_pass.hip), M <= kPassMaxM
// ---------------------------------------------------------------------------
constexpr int kPassMaxM = 16;
constexpr int kPassWaves = 8;  // waves per workgroup
constexpr int kPassRing = 4;   // groups of loads in flight per streaming wave
constexpr int kPassMaxDeps = 4;
// Completion counters: each linear has kPassSub sub-counters, one 64-byte
// line apart; chunk c counts on sub-counter c % kPassSub.  (Atomics on one
// address are performed one at a time: a single counter per linear would
// queue every unit's increment behind the others.)
constexpr int kPassSub = 64;
constexpr int kPassSubStride = 16;  // dwords between sub-counters
// dwords of the counter block of n linears with `arrivals` split chunks: the
// sub-counters, the split chunks' arrival counts, then the exited-workgroup
// count and the error flag
constexpr size_t pass_counter_words(int n, int arrivals) {
    return (size_t)n * kPassSub * kPassSubStride + (size_t)arrivals + 2;
}
// fp32 values of one partial tile of a K-split unit: its rows x 64 columns
constexpr int pass_tile_floats(int M) { return (M == 1 ? 1 : 16) * 64; }

// One linear of a pass, as the kernel reads it (device table).
struct PassLinear {
    const uint16_t* x;   // [M][ldx] bf16, the first K of each row read
    const uint32_t* qt;  // tile layout (w4_repack)
    const uint16_t* st;
    const uint16_t* zt;
    float* y;            // [M][N] fp32, or null
    uint16_t* yb;        // [M][N] bf16, or null
    float alpha;         // output scale
    int N, K, NC, G;     // NC chunks of 64 columns, G groups of 128
    int ldx;             // elements between rows of x
    int unit0;           // the pass's unit number of the linear's first unit (chunk 0, slice 0)
    int kw;              // streaming waves with groups: min(kPassWaves, groups of the smallest slice)
    int ndep;
    int dep[kPassMaxDeps];        // producer linears
    int dep_units[kPassMaxDeps];  // their chunk counts
    int dep_class;       // the first linear with the same set of producers (-1: none)
    int S, gps;          // K slices per chunk (units per chunk) and groups per slice
    int part0, arr0;     // S > 1: first partial tile and first arrival counter of the linear
};

// One launch of the pass kernel.
struct PassLaunch {
    const PassLinear* tab;  // device table
    int n, U, M;            // linears, units, rows
    uint32_t* done;         // sub-counters, then `arrivals` arrival counts
    int arrivals;
    uint32_t* state;        // [0] exited workgroups, [1] error flag
    float* part;            // partial tiles of the K-split units (or null)
    uint32_t spin_limit;
    int grid;
};

hipError_t launch_pass(const PassLaunch& l, hipStream_t stream);

// Workgroups of the pass kernel for M rows that fit one CU at once.
hipError_t pass_occupancy(int M, int* per_cu);

hipError_t launch_bench_read(const void* buf, size_t bytes, uint32_t* sink, int blocks, hipStream_t stream);
hipError_t launch_bench_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);

constexpr int kBenchReadBlocks = 256 * 8;

}  // namespace w4
