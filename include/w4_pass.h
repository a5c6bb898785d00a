/*
 * w4_pass.h -- a whole verify pass of W4A16 linears as one launch.
 *
 * The target model verifies a draft with one forward pass that runs all
 * drafted tokens through every 4-bit linear ("Speculative Decoding Meets
 * Quantization", menfem.com note, Abstract; ordoresearch.ai review,
 * "Research Landscape"), and at plain-decode and sequence-draft sizes that
 * pass is bound by memory bandwidth ("often the primary bottleneck").  A pass
 * object holds the linears of such a pass with their data dependencies; one
 * w4_pass_run launches all of them.  Each linear computes, as w4a16_linear
 * does (include/w4a16.h, same tile layout, same accumulation contract),
 *
 *     y[M][N] = alpha * x[M][K] . dequant(qweight_t, scales_t, zeros_t)
 *
 * and may read, as its x, the output of earlier linears of the pass (its
 * producers, listed in `deps`): its multiply-adds start only once every
 * producer's output is stored, while its weights are already being read.
 *
 * A pass runs in one of two forms.  At M <= 16 it can run as one persistent
 * kernel (one workgroup per CU) that streams the weights of successive
 * linears without a gap between them and runs the linears that share their
 * producers side by side.  At any M it can run each linear as its own
 * launch, in order, on the stream (the same kernels and results as
 * w4a16_linear_out).  w4_pass_create_mode chooses the form (w4_pass_create
 * leaves the choice to the library); w4_pass_info reports it.
 *
 * Conventions are those of include/w4a16.h: device pointers owned by the
 * caller, `stream` a hipStream_t as void*, validation before any HIP call,
 * int status codes, no printing, no aborting.
 */
#ifndef W4_PASS_H
#define W4_PASS_H

#include <stddef.h>
#include <stdint.h>

#include "w4a16.h"

#ifdef __cplusplus
extern "C" {
#endif

/* w4_pass_check: a dependency wait of the last runs gave up (results invalid). */
#define W4_ERR_TIMEOUT 4

#define W4_PASS_MAX_DEPS 4
#define W4_PASS_MAX_LINEARS (1 << 20)

/* One linear of a pass (host struct; pointers are device pointers). */
typedef struct {
    const uint16_t* x;          /* bf16 input: row m at x + m * ldx, its first K values read; 16-byte aligned */
    const uint32_t* qweight_t;  /* tile-layout weights (w4_repack) */
    const uint16_t* scales_t;
    const uint16_t* zeros_t;    /* 4-byte aligned (w4a16_linear needs 2) */
    float* y;                   /* [M][N] fp32 output, or NULL */
    uint16_t* y_bf16;           /* [M][N] bf16 output (round to nearest even), or NULL; at least one output */
    float alpha;                /* output scale (finite; 1 = the plain linear) */
    int N, K;                   /* N % 8 == 0, N >= 8; K % 128 == 0, K >= 128 */
    int ndeps;                  /* 0..W4_PASS_MAX_DEPS */
    int deps[W4_PASS_MAX_DEPS]; /* indices of earlier linears whose outputs must be complete before x is read */
    int ldx;                    /* elements between rows of x: 0 means K; else >= K and a multiple of 8 (so a
                                   linear can read the first K columns of a wider output, e.g. the q part of a
                                   fused q|k|v output) */
} w4_pass_linear;

typedef struct w4_pass w4_pass;

/* Validate the linears of a pass and build a pass object (host call:
 * allocates the device table of the linears and the completion counters on
 * the current device, once, and keeps them until w4_pass_destroy).  `linears`
 * is a host array of n entries; they run in array order at M rows each.
 *
 * Data hazards are checked, never guessed (x counts as the whole span of its
 * M rows, from x to the end of row M - 1's K values): an x that overlaps the output of
 * an earlier linear must list that linear in `deps`; an output may not
 * overlap any input of the same or an earlier linear, any weights, or any
 * other output.  Outputs must be 128-byte aligned and, rounded out to whole
 * 128-byte lines, share no line with any other buffer of the pass other than
 * the inputs that read them (each cache line of an output is written by one
 * linear and read by its consumers only after it is complete).  The buffers
 * must stay allocated, and are not re-checked, until w4_pass_destroy.
 * Returns W4_OK and *out, or W4_ERR_INVALID (null, negative, misaligned,
 * overlapping, a dependency on a later linear, ldx below K or not a
 * multiple of 8), W4_ERR_UNSUPPORTED (group,
 * shapes, M > 64, more than W4_PASS_MAX_DEPS producers) or W4_ERR_HIP. */
int w4_pass_create(const w4_pass_linear* linears, int n, int M, int group, w4_pass** out);

/* The form of a pass (w4_pass_create_mode). */
#define W4_PASS_AUTO 0       /* the library's choice: the persistent kernel at M <= 16 when the linears that share
                                their producers (dependency classes; the linears without producers are one class)
                                number at least 1.25 per class on average, else per-linear launches */
#define W4_PASS_PERSISTENT 1 /* the persistent kernel (M <= 16; W4_ERR_UNSUPPORTED above) */
#define W4_PASS_LAUNCHES 2   /* one launch per linear, in order */

/* w4_pass_create with the form chosen by the caller: `mode` is one of the
 * W4_PASS_* values above (else W4_ERR_INVALID).  Both forms compute the same
 * outputs within the accumulation contract (they may differ in the last
 * bits: the persistent kernel sums a chunk's K range in its own order).
 * Otherwise as w4_pass_create. */
int w4_pass_create_mode(const w4_pass_linear* linears, int n, int M, int group, int mode, w4_pass** out);

/* Launch the whole pass on `stream` (asynchronous).  Allocates nothing and
 * writes no memset: the launch can be captured in a HIP graph and replayed
 * (replays of one pass object on one device must not overlap in time: they
 * share its completion counters).  The inputs may change between runs.
 * Returns W4_OK or W4_ERR_HIP. */
int w4_pass_run(w4_pass* pass, void* stream);

/* Wait for `stream`, then report whether any dependency wait of the runs
 * since the last check gave up (W4_ERR_TIMEOUT: producers never completed --
 * e.g. the device was shared with another kernel that kept some CUs busy --
 * and those runs' outputs are invalid) and clear that flag.  Returns W4_OK,
 * W4_ERR_TIMEOUT, W4_ERR_INVALID (null) or W4_ERR_HIP. */
int w4_pass_check(w4_pass* pass, void* stream);

/* How a pass runs (host outputs, any may be NULL): 1 if it is one persistent
 * launch, else 0 (per-linear launches); that launch's workgroups (0 for
 * launches); its units (the 64-column chunks of all its linears, a chunk
 * that the persistent kernel splits into K slices counting once per slice). */
int w4_pass_info(const w4_pass* pass, int* persistent, int* grid, int* units);

/* Test hook: the number of polls (about 50 ns apart) a dependency wait makes
 * before it gives up and raises the flag w4_pass_check reports; default
 * 2^24 (about a second).  0 makes every wait that is not already satisfied
 * give up at once, which forces the failure path from the host (the launch
 * still runs to its end, its results are invalid).  Returns W4_OK or
 * W4_ERR_INVALID (null). */
int w4_pass_set_spin_limit(w4_pass* pass, uint32_t polls);

/* Free the pass object (device table and counters).  The caller must have
 * synchronized with every run first.  NULL is a no-op. */
int w4_pass_destroy(w4_pass* pass);

#ifdef __cplusplus
}
#endif
#endif /* W4_PASS_H */
