/*
 * w4a16.h -- C ABI of the MI355X (gfx950) W4A16 verify linear.
 *
 * The operation.  Speculative decoding verifies a draft by running the
 * quantised target model once over all drafted tokens ("Speculative
 * Decoding Meets Quantization", menfem.com note and shd-paper.top summary,
 * Abstract; ordoresearch.ai review, "Research Landscape").  In a target
 * with 4-bit weights and 16-bit activations every linear layer of that
 * pass is
 *
 *     y[m, n] = sum_k x[m, k] * (q[k, n] - z[k / g, n]) * s[k / g, n]
 *
 * for the M verified tokens: M = 1 is plain decode, a few rows a sequence
 * draft, tens of rows a flattened tree draft (ordoresearch.ai review,
 * "The Compatibility Problem" and "The Hierarchical Framework").  The pages
 * fix no group size or packing; this library reads them as: uint4 codes q,
 * uint4 zero points z and fp16 scales s per group of g = 128 consecutive k
 * and output column n, bf16 activations x, fp32 output y.
 *
 * Conventions for every entry point.
 *  - Pointers named *device* are device (HBM) pointers owned by the caller;
 *    the library never frees or retains them past the call.  Host pointers
 *    are marked as such.
 *  - `stream` is a hipStream_t passed as void* (NULL = default stream).
 *    Work is enqueued asynchronously on it; results are ready when the
 *    stream has drained.
 *  - Arguments are validated before any HIP call; a failed check returns a
 *    status and launches nothing.  The library never prints or aborts.
 *  - Hidden state: per device, three workspaces allocated together on the
 *    first call that needs one (or by w4_init) and kept until the process
 *    ends -- 64 MiB of split-K partials, 1 MiB for the acceptance step, 48
 *    MiB for tree attention (113 MiB).  A linear with a K split runs as two
 *    launches on the caller's stream (the streaming kernel, then the
 *    reduction of its partials).  Calls that overlap in time on one device
 *    (different streams, or threads) share these workspaces and must not
 *    run concurrently; calls on one stream are ordered by it.
 *    w4a16_linear_out_noalloc uses a static array of its own instead (its
 *    calls must not overlap each other either), and a persistent verify
 *    pass (w4_pass.h, M <= 16) only its own counters.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    W4_OK = 0,
    W4_ERR_INVALID = 1,     /* NULL pointer, negative size, misaligned pointer, y overlapping an input */
    W4_ERR_UNSUPPORTED = 2, /* group != 128, K % 128 != 0, N % 8 != 0, M > 64, size beyond the limits */
    W4_ERR_HIP = 3          /* a HIP call failed (no device, allocation, launch) */
};

/* Largest supported sizes. */
#define W4_MAX_M 64
#define W4_MAX_N (1 << 24)
#define W4_MAX_K (1 << 24)

/* Human-readable name of a status code (static string, never NULL). */
const char* w4_status_str(int status);

/* Detail of the most recent W4_ERR_HIP returned on the calling thread: the
 * failing HIP call and the runtime's error name ("" if none).  Thread-local
 * static storage, valid until the thread's next library call. */
const char* w4_last_error(void);

/* Allocate the split-K workspace of the current device and set kernel
 * attributes now rather than on first use (e.g. before a HIP graph
 * capture).  Idempotent.  Returns W4_OK or W4_ERR_HIP. */
int w4_init(void);

/* Byte sizes of the three arrays w4_repack writes for an (N, K) linear.
 * The tile layout pads N up to a multiple of 64 columns (the padding holds
 * q = z = 0 and s = 0); for N % 64 == 0 the sizes equal the canonical
 * ones: N*K/2, N*K/64 and N*K/256 bytes.  Outputs are host pointers.
 * Returns W4_OK, W4_ERR_INVALID (NULL output, negative size) or
 * W4_ERR_UNSUPPORTED. */
int w4_repacked_sizes(int N, int K, int group, size_t* qweight_bytes, size_t* scales_bytes, size_t* zeros_bytes);

/* Offline repack: canonical packed weights -> gfx950 tile layout.
 *
 * Input (device, canonical format):
 *   qweight int32 [K/8][N]: bits [4i, 4i+4) of word (j, n) hold q[8j+i][n];
 *   scales  uint16 [K/g][N]: fp16 bit patterns;
 *   zeros   int32 [K/g][N/8]: bits [4i, 4i+4) of word (G, j) hold z[G][8j+i].
 * Output (device, sizes from w4_repacked_sizes), NC = ceil(N/64) chunks of
 * 64 columns, KB = K/32 k-blocks, G = K/128 groups:
 *   qweight_t uint32 [NC][KB][64 lanes][4]: word (c, kb, l, j) holds the 8
 *     codes of column 64c + 16j + (l % 16), k = 32kb + 8(l / 16) + e,
 *     e = 0..7, code e at nibble e/2 (e even) or 4 + (e-1)/2 (e odd), the
 *     word then rotated left by 3 bits;
 *   scales_t uint16 [NC][G][16][4]: s[G][64c + 16j + t] at (c, G, t, j),
 *     or 0 where every code of that group and column equals its zero
 *     point (all its weights are 0, so no weight changes; the kernels then
 *     add exactly 0 for it, where the biased sums would leave a rounding
 *     residue unless z = 0);
 *   zeros_t  uint16 [NC][G][16]: nibble j of (c, G, t) is z[G][64c + 16j + t].
 * Not in place; outputs must not overlap inputs.  Stateless. */
int w4_repack(const int32_t* qweight, const uint16_t* scales, const int32_t* zeros, int N, int K, int group,
              uint32_t* qweight_t, uint16_t* scales_t, uint16_t* zeros_t, void* stream);

/* The verify linear:
 *   y[M][N] (device, fp32, row-major, overwritten) =
 *       x[M][K] (device, bf16 bits, row-major) . dequant(qweight_t, scales_t, zeros_t)
 * with the tile-layout arrays from w4_repack.  0 <= M <= 64; M == 0 or
 * N == 0 does nothing; K == 0 writes y = 0.  Alignment: x, qweight_t and y
 * 16 bytes, scales_t 8, zeros_t 2.  y must not overlap any input.
 * Accumulation is fp32; each element is within 4e-3 * sum_k |x w| of the
 * exact value (in practice orders of magnitude closer).  The result does
 * not depend on the stream or on other calls.  M == 1 runs the VALU dot
 * (GEMV) kernel, M >= 2 the bf16 MFMA kernel. */
int w4a16_linear(const uint16_t* x, const uint32_t* qweight_t, const uint16_t* scales_t, const uint16_t* zeros_t,
                 int M, int N, int K, int group, float* y, void* stream);

/* Kernel choice for w4a16_linear_cfg. */
enum { W4_KERNEL_AUTO = 0, W4_KERNEL_GEMV = 1, W4_KERNEL_MFMA = 2 };

/* w4a16_linear with the launch plan forced, for tests and tuning sweeps.
 * kernel: W4_KERNEL_*; GEMV needs M == 1.  splits: number of K splits
 * (0 = automatic), clamped to [1, K/128] and to what the workspace and LDS
 * allow.  Same result contract as w4a16_linear. */
int w4a16_linear_cfg(const uint16_t* x, const uint32_t* qweight_t, const uint16_t* scales_t,
                     const uint16_t* zeros_t, int M, int N, int K, int group, float* y, int kernel, int splits,
                     void* stream);

/* Output element types for w4a16_linear_out. */
enum { W4_OUT_F32 = 0, W4_OUT_BF16 = 1 };

/* w4a16_linear_cfg with a choice of output type.  W4_OUT_F32: y is fp32, as
 * in w4a16_linear.  W4_OUT_BF16: y (device, 16-byte aligned, M*N uint16
 * bf16 bit patterns, row-major) receives the fp32 result rounded to nearest,
 * ties to even -- bit for bit what rounding w4a16_linear_cfg's fp32 output
 * with the same kernel and split count would give; half the output bytes,
 * and the activation type the next layer consumes.  The pages leave the
 * output type open; this is the bf16 epilogue of the fused-projection
 * follow-up (qkv as one N = 10240 linear, gate|up as N = 57344: the tile
 * layout of a column concatenation is the concatenation of the parts' tile
 * layouts when every part's N is a multiple of 64).  Other out_dtype values:
 * W4_ERR_INVALID. */
int w4a16_linear_out(const uint16_t* x, const uint32_t* qweight_t, const uint16_t* scales_t,
                     const uint16_t* zeros_t, int M, int N, int K, int group, void* y, int out_dtype, int kernel,
                     int splits, void* stream);

/* w4a16_linear_out for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, plans, kernels and result (bit for bit) as w4a16_linear_out,
 * but the split-K partials go to a static device array of 64 MiB per GPU
 * (W4_NOALLOC_SCRATCH_BYTES) that the library holds from module load until
 * the process ends, instead of the lazily allocated workspace: the call
 * makes no hipMalloc, hipFree or other allocating call.  The first call on
 * a device looks the array's address up (hipGetSymbolAddress) and keeps it.
 * A forced `splits` whose partials (splits * M * ceil(N/64)*64 fp32) would
 * not fit the array returns W4_ERR_UNSUPPORTED; splits = 0 always fits.
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one device (different streams) race and may return wrong results.  The
 * array needs no clearing (every partial a call reads, it first writes). */
#define W4_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int w4a16_linear_out_noalloc(const uint16_t* x, const uint32_t* qweight_t, const uint16_t* scales_t,
                             const uint16_t* zeros_t, int M, int N, int K, int group, void* y, int out_dtype,
                             int kernel, int splits, void* stream);

/* w4a16_linear_out with the work decomposition of the M <= 16 kernels
 * forced as well, for tests and tuning sweeps.  kwaves: 0 = automatic (at
 * M = 15, 16 with N >= 4096 the LDS-ring kernel of M > 16, one chunk per
 * wave); any other value keeps M <= 16 on the streaming MFMA kernel; 1 =
 * each wave of a workgroup streams its own 64-column chunk (four per
 * workgroup) over the workgroup's K split; 2, 4 or 8 = a workgroup of that
 * many waves streams one chunk, its waves splitting the K split's groups and
 * summing their parts in LDS (no split-K workspace when splits is 1).
 * Reduced when the smallest K split has fewer groups than waves; kwaves > 1
 * with M > 16, or not 0/1/2/4/8: W4_ERR_UNSUPPORTED, negative:
 * W4_ERR_INVALID.  Same result contract as w4a16_linear. */
int w4a16_linear_tune(const uint16_t* x, const uint32_t* qweight_t, const uint16_t* scales_t,
                      const uint16_t* zeros_t, int M, int N, int K, int group, void* y, int out_dtype, int kernel,
                      int splits, int kwaves, void* stream);

/* The launch plan w4a16_linear_tune would use for (kernel, splits, kwaves)
 * (host outputs, any may be NULL): kernel id, K splits, waves splitting a
 * chunk's K range, workgroups, threads per workgroup, LDS bytes per
 * workgroup.  With kwaves 1 each wave streams its own chunk and the
 * workgroup holds threads/64 of them: four, or in the LDS-ring kernel
 * (lds_out > 0: M > 16, or M = 15, 16 with N >= 4096 and kwaves 0) four or
 * eight (the planner's choice, also when splits is forced).  Workgroups =
 * column tiles x K splits x row slices: the LDS-ring kernel shares the row
 * blocks of a narrow linear out between two to four workgroups (row slices)
 * where even its most splits would leave half of the 256 CUs idle; the
 * slice count is grid_out / (tiles x splits).  No HIP call. */
int w4a16_plan(int M, int N, int K, int group, int kernel, int splits, int kwaves, int* kernel_out,
               int* splits_out, int* kwaves_out, int* grid_out, int* block_out, int* lds_out);

/* One linear of a verify pass (host struct; pointers are device). */
typedef struct {
    const uint16_t* x;         /* [M][K] bf16 input */
    const uint32_t* qweight_t; /* tile-layout weights */
    const uint16_t* scales_t;
    const uint16_t* zeros_t;
    float* y;                  /* [M][N] fp32 output */
    int N, K;
} w4_linear_desc;

/* A whole verify pass: every linear of the target model at the same M, in
 * array order, on one stream (the target's single batched forward over
 * the draft, ordoresearch.ai review "Research Landscape").  `linears` is a
 * host array of n entries; all are validated before the first launch.
 * Capturable in a HIP graph once the workspace exists (w4_init). */
int w4a16_verify_pass(const w4_linear_desc* linears, int n, int M, int group, void* stream);

/* Test-only: tile layout -> canonical bytes through the kernels' own unpack
 * path.  q_out uint8 [K][N] (device) gets q[k][n]; z_out uint8 [K/g][N]
 * (device) gets z[G][n].  Bit-exact inverse of w4_repack on the codes. */
int w4_unpack(const uint32_t* qweight_t, const uint16_t* zeros_t, int N, int K, int group, uint8_t* q_out,
              uint8_t* z_out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* W4A16_H */
