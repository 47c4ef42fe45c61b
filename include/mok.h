/*
 * mok.h -- C ABI of a deterministic mixture-of-experts layer for AMD MI355X
 * (gfx950 / CDNA4).
 *
 * The layer routes each of T tokens to k of E experts, runs every routed row
 * through its expert's SwiGLU FFN and adds the k expert outputs back with the
 * router's combine weights; its backward returns the gradients of the input,
 * of every expert weight and of the combine weights. Sources, cited by title
 * and section:
 *   [MoK card] "Mixture-Of-Kittens (MoK)" project card (agentlenshq.com):
 *              "What it is", "Using the functional API", "Core concepts".
 *   [MoK clip] "Mixture-of-Kittens: Cursor open-sources an MoE training
 *              megakernel" (miguoliang.com clip): "Key points", "How to",
 *              and the key chart.
 *   [OCP MX]   OCP Microscaling Formats (MX) Specification v1.0.
 *
 * Conventions for every call
 *   - Pointers are DEVICE pointers unless marked [host]. `stream` is a
 *     hipStream_t passed as void* (NULL = the default stream).
 *   - Calls that take a stream only enqueue work on it: they never
 *     synchronize the host with the device, never allocate memory and never
 *     read device memory from the host ([MoK clip] Key points, bullet 4:
 *     routing counts stay on the device).
 *   - The caller owns and allocates every buffer (sizes from
 *     mok_buffer_sizes) and keeps it alive until the enqueued work is done.
 *     Inputs and outputs must not alias. The library keeps no per-call state.
 *   - Outputs are overwritten, never accumulated into.
 *   - Errors found on the host return a negative mok_status before anything
 *     is enqueued. Errors that only the device can see (an expert id outside
 *     [0, E)) set a bit in the schedule's status word instead; the rows
 *     concerned are skipped without any out-of-bounds access.
 *   - Results are bitwise reproducible: the same inputs, problem, config and
 *     device give the same output bytes on every call ([MoK clip] How-to
 *     item 6: a fixed floating-point accumulation order).
 *
 * Layouts (row-major, bf16 = IEEE bfloat16 bit patterns)
 *   topk_ids  [T][k] int32      expert of pick j of token t; flat row i = t*k + j
 *   topk_w    [T][k] float32    combine weight of pick j (used as given)
 *   x, y, dy, dx  [T][H] bf16
 *   w_gate, w_up  [E][I][H]     bf16, or E4M3 codes (MXFP8)
 *   w_down        [E][H][I]     bf16, or E4M3 codes (MXFP8)
 *   s_gate, s_up  [E][I][H/32]  E8M0 scale bytes (MXFP8 only)
 *   s_down        [E][H][I/32]  E8M0 scale bytes (MXFP8 only)
 * The expert FFN is h = silu(x Wg^T) * (x Wu^T), out = h Wd^T, no biases.
 */
#ifndef MOK_H
#define MOK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOK_OK = 0,
  MOK_ERR_INVALID_ARG = -1,      /* null pointer, bad size or shape            */
  MOK_ERR_UNSUPPORTED = -2,      /* valid but not supported by this library    */
  MOK_ERR_BUFFER_TOO_SMALL = -3, /* a caller buffer is below mok_buffer_sizes  */
  MOK_ERR_DEVICE = -4            /* no gfx950 device, or a launch failed       */
} mok_status;

typedef enum { MOK_BF16 = 0, MOK_MXFP8 = 1 } mok_dtype;

/* Status word bits, written by mok_build_schedule (and the second by
 * mok_forward with driver 2 and by mok_forward_fused); read the word after
 * the stream has passed the call. */
#define MOK_STATUS_BAD_EXPERT_ID 0x1   /* some topk_ids value was outside [0, E) */
#define MOK_STATUS_WATCHDOG      0x2   /* driver 2 gave up: a wait between its
                                          tiles passed its time limit (2 s; the
                                          environment variable
                                          MOK_PERSIST_SPIN_TICKS=n sets it to n
                                          ticks of the 100 MHz counter, for
                                          tests), or the schedule's tile table
                                          failed its checks; y and fwd_ctx are
                                          incomplete. Set by mok_forward
                                          (driver 2) and mok_forward_fused.     */

/* Problem shape. Supported: T >= 0, 1 <= topk <= E <= 512, T*topk < 2^31,
 * H and I multiples of 128. dtype MOK_MXFP8 selects the MXFP8 forward and
 * backward (weights pre-quantized, see mok_weights). */
typedef struct {
  int64_t T, H, I;
  int32_t E, topk;
  int32_t dtype;                 /* mok_dtype */
} mok_problem;

/* Tuning knobs ([MoK card] "Core concepts": minibatch granularity,
 * macrobatch size, schedule capacity multiplier; the communication-CU count
 * has no meaning on one GPU and is not present). Zero selects the default. */
typedef struct {
  int32_t minibatch_rows;        /* M, routed rows per minibatch. Default:
                                    [MoK clip] How-to item 3 asks that each
                                    grouped GEMM fill two waves (M >= 4*S*H/I for
                                    its tiles); for this library's 256x256 tiles
                                    that is M >= S*65536/I. Default
                                    M = round_up(max(4*S*H/I, S*65536/I), 256),
                                    capped at T*topk.                            */
  int32_t ring_slots;            /* N_s, slots of the ring token buffer (the
                                    "macrobatch" is N_s*M rows). Default 4,
                                    capped at the minibatch count.               */
  float capacity_multiplier;     /* accepted (0 or >= 1); on one GPU the exact
                                    row count T*topk is always used.              */
  int32_t num_cus;               /* S for the default M; 0 = 256 (MI355X).        */
  int32_t driver;                /* 0 = default (= 1), 1 = one launch per
                                    stage (gate/up, down) per ring group of
                                    N_s minibatches,
                                    2 = one persistent launch for all minibatches:
                                    a resident grid takes the gate/up and down
                                    tiles from per-XCD queues, minibatch after
                                    minibatch, the tiles waking each other
                                    through device counters and a ring slot
                                    reused once the down tiles that read it
                                    are done ([MoK clip] Key points 3-5).
                                    Results are bitwise those of driver 1.
                                    Runs alone on the device: kernels of other
                                    streams that hold CUs for long can make its
                                    waits give up (MOK_STATUS_WATCHDOG).       */
} mok_config;

typedef struct {
  const void* w_gate;            /* [E][I][H] */
  const void* w_up;              /* [E][I][H] */
  const void* w_down;            /* [E][H][I] */
  const uint8_t* s_gate;         /* MXFP8 only, else NULL */
  const uint8_t* s_up;
  const uint8_t* s_down;
  /* MXFP8 backward only (else NULL): the weights quantized along the other
   * axis, for the GEMMs that contract over I or H of their output side:
   * w_down_t = Wd^T [E][I][H] E4M3 with s_down_t [E][I][H/32] (blocks along H);
   * w_gu_t = [Wg; Wu]^T [E][H][2I] E4M3 with s_gu_t [E][H][2I/32] (blocks
   * along 2I; I is a multiple of 32, so no block spans Wg and Wu). Both come
   * from mok_mxfp8_quantize_transposed of the bf16 weights (Wd with ld = H;
   * Wg at col0 = 0 and Wu at col0 = I with ld = 2I). */
  const void* w_down_t;
  const void* w_gu_t;
  const uint8_t* s_down_t;
  const uint8_t* s_gu_t;
} mok_weights;

/* Byte offsets of the arrays inside the schedule buffer (each 256-aligned). */
typedef struct {
  size_t status;                 /* int32 status word                              */
  size_t counts;                 /* int32 [E]   rows routed to each expert         */
  size_t offsets;                /* int32 [E+1] exclusive prefix sum of counts;
                                    offsets[E] = number of valid rows              */
  size_t perm;                   /* int32 [R]   flat row at permuted position p    */
  size_t dest;                   /* int32 [R]   permuted position of flat row i    */
  size_t n_fwd_tiles;            /* int32       forward row tiles                  */
  size_t fwd_tiles;              /* int32x4 [max_fwd_tiles] {e, p0, p1, m}          */
  size_t mb_tile_start;          /* int32 [n_minibatches + 1]                      */
  size_t n_bwd_tiles;            /* int32       backward row tiles                 */
  size_t bwd_tiles;              /* int32x4 [max_bwd_tiles] {e, p0, p1, 0}          */
  size_t total;                  /* buffer size; the bytes after bwd_tiles are
                                    scratch of mok_build_schedule              */
  int32_t minibatch_rows;        /* resolved M   */
  int32_t ring_slots;            /* resolved N_s */
  int32_t n_minibatches;         /* ceil(R / M)  */
  int32_t max_fwd_tiles, max_bwd_tiles, fwd_tile_rows, bwd_tile_rows;
  size_t arrays;                 /* bytes of the schedule arrays alone, without the
                                    build's scratch tail: the size
                                    mok_build_schedule_noalloc needs              */
  size_t expert_order;           /* int32 [E]   experts by descending count, ties
                                    to the lower id (the order in which the
                                    weight-gradient GEMMs take the experts)       */
} mok_schedule_layout;

/* [host] Library version, major*10000 + minor*100 + patch. */
int32_t mok_version(void);

/* [host] Static text for a status code. */
const char* mok_status_string(int32_t status);

/* [host] Sizes in bytes of the three caller-allocated buffers for `problem`
 * under `config` (NULL = defaults). No device access. workspace: scratch for
 * any call, reusable across layers. schedule: written by mok_build_schedule,
 * read by forward and backward. fwd_ctx: what forward saves for backward
 * ([MoK card] "Using the functional API": forward returns (out, fwd_ctx)). */
mok_status mok_buffer_sizes(const mok_problem* problem, const mok_config* config,
                            size_t* workspace_bytes, size_t* schedule_bytes,
                            size_t* fwd_ctx_bytes);

/* [host] Where each schedule array lives inside the schedule buffer. */
mok_status mok_get_schedule_layout(const mok_problem* problem, const mok_config* config,
                                   mok_schedule_layout* layout);

/* Routing schedule ([MoK card] "Using the functional API": build_schedule
 * from the top-k expert choices; [MoK clip] Key points, bullet 4: built
 * entirely on the GPU; How-to item 2: one schedule serves all four exchange
 * passes of forward and backward).
 * Computes per-expert counts, their exclusive prefix sum, and the stable
 * permutation of the T*k routed rows into expert order (ties by flat row
 * index), its inverse, and the row tiles of the grouped GEMMs: forward tiles
 * never cross an expert or a minibatch boundary (minibatch m = permuted rows
 * [m*M, (m+1)*M), held in ring slot m mod N_s). Rows whose id is outside
 * [0, E) are placed after every valid row and set MOK_STATUS_BAD_EXPERT_ID. */
mok_status mok_build_schedule(const mok_problem* problem, const mok_config* config,
                              const int32_t* topk_ids,
                              void* schedule, size_t schedule_bytes, void* stream);

/* The same schedule for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): identical results to mok_build_schedule, but the build's
 * scratch (the per-chunk count table) lives in a static device array of the
 * library instead of the tail of `schedule`, so schedule_bytes need only be
 * mok_schedule_layout's `arrays` (passing the full size is fine too).
 * The array holds 2048 x 513 x 4 bytes (about 4 MiB), one copy per GPU,
 * kept until the process ends; it covers every supported problem, and a
 * problem needing more returns MOK_ERR_UNSUPPORTED. Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (other streams,
 * other host threads) race and must not run concurrently. Allocates nothing:
 * no hipMalloc, no library allocation. Errors as mok_build_schedule, plus
 * MOK_ERR_DEVICE if the array's device address cannot be obtained. */
mok_status mok_build_schedule_noalloc(const mok_problem* problem, const mok_config* config,
                                      const int32_t* topk_ids, void* schedule, size_t schedule_bytes,
                                      void* stream);

/* Forward ([MoK clip] Conclusion and key chart: dispatch -> expert SwiGLU
 * FFN -> combine -> weighted sum). Per minibatch, in order: gate/up grouped
 * GEMM over the rows x[perm[p] / k] (the dispatch: the GEMM reads them in
 * place), with the SwiGLU in its epilogue writing h to a ring slot; down
 * grouped GEMM writing each expert output to its flat row i; then
 * y[t] = sum_{j=0..k-1} topk_w[t][j] * out[t*k + j], accumulated in fp32 in
 * ascending j and rounded once to bf16.
 * fwd_ctx: NULL for inference; else receives what mok_backward needs: the
 * expert outputs and the gate/up pre-activations (bf16). MXFP8 ([MoK card]
 * "Core concepts": weights pre-quantized with mok_mxfp8_quantize): x rows are
 * quantized along H (once per token) and h along I the same way on the fly;
 * accumulation is fp32, y is bf16. x, topk_w and y may be NULL when T = 0
 * (nothing is read or written). With config->driver == 2 the call may set
 * MOK_STATUS_WATCHDOG in the schedule's status word (the only write to the
 * schedule). */
mok_status mok_forward(const mok_problem* problem, const mok_config* config,
                       const void* schedule, const void* x, const float* topk_w,
                       const mok_weights* weights, void* y, void* fwd_ctx,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Single-launch forward ([MoK card] "What it is": the layer in one kernel;
 * [MoK clip] Key points 4-5 and key chart: schedule generation on the GPU,
 * then dispatch -> expert FFN -> combine, stages waking each other through
 * device counters). One persistent grid (a workgroup per compute unit) builds
 * the schedule from topk_ids (the steps of mok_build_schedule), runs the
 * minibatch forward of driver 2 (the dispatch fused into the gate/up operand
 * copies, the down rows pushed to their flat slots) and the weighted combine;
 * a small fill kernel clears its counters first, on the same stream.
 * Arguments: those of mok_build_schedule (topk_ids, schedule, schedule_bytes:
 * the schedule written is the one mok_build_schedule writes, so mok_backward
 * can use it) and of mok_forward (x, topk_w, weights, y, fwd_ctx, workspace);
 * config->driver is ignored. Results: schedule, y and fwd_ctx bitwise those of
 * mok_build_schedule followed by mok_forward. The grid waits for itself
 * between steps, so it must have the device to itself: kernels of other
 * streams that hold compute units can make a wait give up after 2 s, which
 * sets MOK_STATUS_WATCHDOG in the schedule's status word and leaves y and
 * fwd_ctx incomplete. Errors as mok_build_schedule and mok_forward, plus
 * MOK_ERR_UNSUPPORTED where the item counts would overflow 32-bit tickets. */
mok_status mok_forward_fused(const mok_problem* problem, const mok_config* config,
                             const int32_t* topk_ids, void* schedule, size_t schedule_bytes,
                             const void* x, const float* topk_w, const mok_weights* weights,
                             void* y, void* fwd_ctx, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Backward. [MoK clip] How-to item 2: reverse-combine then reverse-dispatch
 * with the same schedule; [MoK card] "What it is": forward and backward in
 * BF16 and MXFP8. x and dy rows are read in place through the schedule
 * (x must be the forward's input). MXFP8 (fwd_ctx from an MXFP8
 * forward, weights with the transposed copies of mok_weights): every
 * backward GEMM takes MXFP8 operands blocked by 32 along its contraction
 * axis -- dO along H, dA|dB along 2I, and for the weight gradients dO, h,
 * dA|dB and x along each expert's rows in blocks counted from its first
 * permuted row; accumulation fp32, outputs bf16 / fp32 as below. Outputs:
 *   d_topk_w[t][j] = <dy[t], out[t*k+j]>           (fp32)
 *   dx [T][H], dw_gate/dw_up [E][I][H], dw_down [E][H][I]   (bf16)
 * Every reduction runs in a fixed order with no atomics; an expert with no
 * rows gets exact-zero weight gradients. fwd_ctx, x, topk_w, dy, dx and
 * d_topk_w may be NULL when T = 0 (then every weight gradient is zero). */
mok_status mok_backward(const mok_problem* problem, const mok_config* config,
                        const void* schedule, const void* fwd_ctx,
                        const void* x, const float* topk_w, const mok_weights* weights,
                        const void* dy, void* dx, void* dw_gate, void* dw_up,
                        void* dw_down, float* d_topk_w,
                        void* workspace, size_t workspace_bytes, void* stream);

/* MXFP8 quantization ([MoK card] "Core concepts" and "Limits": MXFP8
 * weights are pre-quantized by an op; block format from [OCP MX]).
 * src [rows][K] bf16 -> q [rows][K] E4M3 codes and scales [rows][K/32] E8M0:
 * per 32-element block, s = clamp(floor(log2 amax) - 8 + 127, 0, 254)
 * (0 for an all-zero block) and q = E4M3(v * 2^(127-s)), round to nearest
 * even, saturating at 448. K must be a multiple of 32; rows >= 0. */
mok_status mok_mxfp8_quantize(const void* src, int64_t rows, int64_t K,
                              uint8_t* q, uint8_t* scales, void* stream);

/* MXFP8 quantization along the other axis ([MoK card] "Core concepts" and
 * "Limits": pre-quantized MXFP8 weights; the MXFP8 backward contracts the
 * weights over their output axis, so it needs copies blocked along that axis).
 * src [batch][rows][cols] bf16 -> q[b][c][col0 + r] = E4M3 code of src[b][r][c]
 * and scales[b][c][(col0 + r)/32], blocked by 32 along r: exactly the codes and
 * scale bytes mok_mxfp8_quantize gives for each transposed [cols][rows] matrix,
 * written into columns [col0, col0 + rows) of a [cols][ld] output (other
 * columns untouched), so that two calls can fill [Wg; Wu]^T.
 * q is [batch][cols][ld] bytes, scales [batch][cols][ld/32] bytes.
 * Requires rows, ld and col0 multiples of 32, cols a multiple of 8,
 * col0 + rows <= ld, src and q 16-byte aligned (MOK_ERR_INVALID_ARG
 * otherwise); batch <= 65535 (MOK_ERR_UNSUPPORTED). Empty inputs are a no-op. */
mok_status mok_mxfp8_quantize_transposed(const void* src, int64_t batch, int64_t rows, int64_t cols,
                                         uint8_t* q, uint8_t* scales, int64_t ld, int64_t col0,
                                         void* stream);

/* ---------------------------------------------------------------- router
 * Router front end ([MoK clip] key chart: "Router picks top-k", upstream of
 * the layer; the pages give no formula, this is the plainest reading):
 *   logits[t][e] = sum_h x[t][h] * w_router[e][h]   (fp32, fixed order:
 *   on the matrix cores, with w_router split exactly into three bf16 parts
 *   so that every product is exact)
 *   score = logit + bias[e] (bias optional, NULL = none; it moves the
 *   selection only), topk_ids[t] = the k largest scores in descending
 *   order, equal scores in ascending expert id, and
 *   topk_w[t][j] = softmax over the k selected (unbiased) logits, fp32.
 * x [T][H] bf16, w_router [E][H] fp32 (device), bias [E] fp32 or NULL;
 * outputs topk_ids [T][k] int32 and topk_w [T][k] fp32, overwritten.
 * Requires k <= 64 (one wavefront holds the picks): MOK_ERR_UNSUPPORTED
 * otherwise. NaN logits are not supported. */
mok_status mok_router_forward(const mok_problem* problem, const void* x, const float* w_router,
                              const float* bias, int32_t* topk_ids, float* topk_w, void* stream);

/* Router backward from g = d topk_w [T][k] (fp32): the selection is held
 * fixed, so only the selected logits get gradient, through the softmax:
 *   d_sel[t][j] = w_j * (g_j - sum_i w_i g_i)               [T][k] fp32
 *   dx[t] = sum_j d_sel[t][j] * w_router[topk_ids[t][j]]     [T][H] bf16
 *   d_w_router[e] = sum over the rows routed to e of d_sel * x[t]   [E][H] fp32
 * (the caller adds dx to the layer's dx). schedule is the one built by
 * mok_build_schedule for these topk_ids (its permutation orders the dWr
 * sums: each expert's rows in 4 fixed interleaved groups of ascending rows,
 * added in group order; an expert with no rows gets exact zeros). Ids
 * outside [0, E) contribute nothing. All outputs are overwritten. */
mok_status mok_router_backward(const mok_problem* problem, const mok_config* config, const void* schedule,
                               const void* x, const float* w_router, const int32_t* topk_ids,
                               const float* topk_w, const float* d_topk_w, float* d_sel, void* dx,
                               float* d_w_router, void* stream);

/* ---------------------------------------------------------------- tracing
 * Per-kernel timing for profiling ([MoK clip] How-to item 1: profile first to
 * see where the layer's time goes). While tracing is on, every kernel the
 * library launches is bracketed by two HIP events recorded on its launch
 * stream (host-side calls only; nothing waits; timing-only events created
 * with hipEventDisableSystemFence, so they add no cache writeback between
 * kernels). mok_trace_collect synchronises the device and reads the recorded
 * events (a host synchronisation, so never call it inside a
 * timed or captured region), returns per-kernel totals in launch order of
 * first appearance and clears the record. The library creates and reuses
 * the events itself. Not thread-safe across concurrent callers. */
typedef struct {
  char name[40];
  int32_t launches;
  double total_ms;
  double max_ms;
} mok_trace_stat;

/* [host] on != 0 starts recording, 0 stops (records are kept until collected). */
mok_status mok_trace_enable(int32_t on);

/* [host] Fill out[0 .. min(n, capacity)) and *n_out = n, the number of kernels. */
mok_status mok_trace_collect(mok_trace_stat* out, int32_t capacity, int32_t* n_out);

/* ---------------------------------------------------------------- peak probe
 * Matrix-core rate the device sustains, for putting the grouped GEMMs' rates
 * beside a measured peak ([MoK clip] How-to item 1: profile first). Enqueues
 * `workgroups` workgroups of 4 wavefronts; each wavefront issues 8 * iters
 * matrix instructions back to back on register operands (no memory traffic):
 * kind 0 = bf16 (v_mfma_f32_32x32x16_bf16, 32768 FLOP each), kind 1 = MXFP8
 * (v_mfma_scale_f32_32x32x64_f8f6f4 on E4M3, 131072 FLOP each). Total FLOP =
 * workgroups * 4 * 8 * iters * (FLOP each). Writes one float per thread to
 * sink [workgroups * 256] (device). The caller times it on `stream`. Kind not
 * 0 or 1, negative counts, or a NULL sink with work to do: MOK_ERR_INVALID_ARG. */
mok_status mok_probe_mfma(int32_t kind, int32_t workgroups, int32_t iters, float* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOK_H */
