/*
 * exl3.h -- C ABI of the MI355X (gfx950) EXL3 quantized linear.
 *
 *     y = had( W_q . had(x * suh) ) * svh
 *
 * W_q is decoded on the fly from 16x16 trellis tiles; it is never stored.
 *
 * Sources (the pages this library implements):
 *   - cuda-exl3 README, "One op per layer": one call does a whole quantized
 *     linear; all shards of a fused layer run in one GEMM, addressed by
 *     absolute column; the output is in the caller's dtype (bf16 or fp16); the
 *     activation transform is a separate kernel ("Two further departures").
 *   - cuda-exl3 README, "Notes on the format": suh has one row per shard,
 *     trellis and svh concatenate along the output dim.
 *   - TensorFold PR "cuda: EXL3 projections behind qlinear", "What it adds":
 *     trellis [K/16][N/16][16*bits] int16, widths 1..8, codebooks 3inst, mcg
 *     and mul1; "Arithmetic": the rounding order (x*suh, fp32 Hadamard,
 *     *2^-4, one rounding to fp16; fp16 products with fp32 sums; output
 *     Hadamard, svh and 2^-3, one rounding); a shape-fixed number of K parts
 *     summed in part order, so a row's bits do not depend on the batch.
 *
 * Conventions for every call
 *   - Pointers are DEVICE pointers unless marked HOST.  The caller owns every
 *     buffer and the stream; no call allocates, frees or synchronizes, so all
 *     calls may be captured in a HIP graph.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued asynchronously on it.
 *   - Every argument is validated on the host before any HIP call.  On error
 *     nothing is enqueued or written, the status is returned, and
 *     exl3_last_error() names the failed check and the offending values.
 *   - Device pointers must be 16-byte aligned.  Matrices are row-major and
 *     dense (no strides).  fp16/bf16 data are passed as raw uint16 bits.
 *   - Shapes: K and every shard width are multiples of 128 (the Hadamard
 *     block); bits in 1..8; 1..EXL3_MAX_SHARDS shards; M >= 0 (M == 0 is a
 *     no-op that returns EXL3_OK).
 *   - Calls on distinct outputs and workspaces may run concurrently.
 */
#ifndef EXL3_H
#define EXL3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EXL3_MAX_SHARDS 16
#define EXL3_ABI_VERSION 6

/* The first EXL3_WORKSPACE_COUNTER_BYTES of every workspace hold per-tile
 * arrival counters (see exl3_linear): they must be zero before the first
 * call that uses the workspace, and every call leaves them zero. */
#define EXL3_WORKSPACE_COUNTER_BYTES 65536

typedef enum {
  EXL3_OK = 0,
  EXL3_ERR_INVALID_ARG = 1, /* a shape, pointer, alignment or enum is wrong  */
  EXL3_ERR_UNSUPPORTED = 2, /* valid EXL3, but outside this build's limits   */
  EXL3_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required    */
  EXL3_ERR_LAUNCH = 4       /* the HIP runtime refused a launch              */
} exl3_status;

/* The three procedural codebooks (cuda-exl3 README, "What is supported"). */
typedef enum { EXL3_CB_3INST = 0, EXL3_CB_MCG = 1, EXL3_CB_MUL1 = 2 } exl3_codebook;

typedef enum { EXL3_F16 = 0, EXL3_BF16 = 1 } exl3_dtype;

/* One EXL3 weight, possibly a fused multi-shard layer (qkv, gate_up).
 * The weight view of the TensorFold PR ("What it adds") plus the shard map
 * of the cuda-exl3 README ("One op per layer", "Notes on the format"). */
typedef struct exl3_weight {
  const uint16_t *trellis; /* [K/16][N/16][16*bits] trellis words           */
  const uint16_t *suh;     /* fp16 bits [n_shards][K], one row per shard     */
  const uint16_t *svh;     /* fp16 bits [N], absolute output column          */
  int32_t K;               /* input features, multiple of 128                */
  int32_t N;               /* output features = sum(shard_n)                 */
  int32_t bits;            /* 1..8 bits per weight                           */
  int32_t codebook;        /* exl3_codebook                                  */
  int32_t n_shards;        /* 1..EXL3_MAX_SHARDS                             */
  const int32_t *shard_n;  /* HOST [n_shards], each a multiple of 128        */
  const uint16_t *bias;    /* fp16 bits [N] or NULL: the format's bias
                              (cuda-exl3 README, "VRAM"), added in fp32 to
                              svh * 2^-3 * H128(z) before the one rounding    */
} exl3_weight;

/* Execution plan.  `parts` (P), `groups` (G) and the K range of each part
 * depend on (K, N, bits) only, never on M, so every row's result is
 * bit-identical at every batch size.  The fp32 sum over K is the fixed tree:
 * each part is one chain of matrix-core products in ascending k starting from
 * zero; the P/G consecutive parts of a group are added in part order (first
 * part copied); the group sums are added in group order (first copied).  With
 * G == P this is the plain ((p0 + p1) + p2) + ... of the TensorFold PR
 * ("Arithmetic": a number of parts fixed by the shape, added by the last
 * part in part order).  G < P, the two-level grouping that small layers
 * get, is this library's own choice, fixed by the shape like P.  `mode`,
 * `bm`, `decoder` and `unit` pick how the same arithmetic is scheduled and
 * never change a bit of the output. */
typedef enum {
  EXL3_MODE_AUTO = -1,
  EXL3_MODE_FUSED = 0, /* one workgroup per (M-tile, 128 columns) runs all
                          parts in order and applies the output transform
                          (one group, or one part per group)                */
  EXL3_MODE_SLABS = 1  /* one workgroup per (M-tile, 128 columns, unit of
                          parts) writes the unit's fp32 sum as a partial
                          slab; the slabs are summed in order and the output
                          transform applied by the tile's last workgroup
                          (the finisher) or by a second kernel              */
} exl3_mode;

/* How weights are decoded.  Both decoders produce the same fp16 values
 * (the table is filled by the ALU decoder) and run the same MFMA chains. */
typedef enum {
  EXL3_DECODER_AUTO = -1,
  EXL3_DECODER_ALU = 0,  /* tile kernels (bm rows per workgroup): every
                            weight decoded by vector ALU instructions        */
  EXL3_DECODER_TABLE = 1, /* M <= 64 only: one persistent 1024-thread
                            workgroup per CU fills a 65,536-entry state ->
                            fp16 table in LDS and decodes half of the
                            weights through it, the rest by the ALU (512
                            threads above 32 rows)                           */
  EXL3_DECODER_DENSE = 2 /* large batches: the whole W_q is decoded once
                            into the workspace (K*N fp16, as matrix-core
                            operand fragments), then a dense GEMM in
                            256-row tiles reads it; same bits             */
} exl3_decoder;

typedef struct exl3_plan {
  int32_t parts;       /* P >= 1 K parts, all of whole 128-k blocks          */
  int32_t groups;      /* G >= 1 groups, G divides P; when P/G > 1 every
                          part has the same length (P divides K/128)        */
  int32_t mode;        /* exl3_mode                                          */
  int32_t bm;          /* rows per M-tile: 16, 32, 64, 128, 256 or 512;
                          512 only with one part per workgroup (parts == 1
                          or slab mode), else EXL3_ERR_UNSUPPORTED.  The
                          table decoder reports 16, 32 or 64                */
  int32_t decoder;     /* exl3_decoder.  Automatic: TABLE for M <= 64 on
                          layers of at least 2^25 weights (2^26 when
                          M <= 16) and at most 2 GiB of trellis, DENSE
                          for M >= 2048 on layers
                          of at least 2^25 weights, else ALU.  In a
                          forced plan 0 means ALU; TABLE with M > 64 is
                          EXL3_ERR_UNSUPPORTED; forcing bm alone selects
                          ALU.  DENSE runs 256-row tiles                     */
  int32_t unit;        /* slab mode: parts per workgroup unit (one slab per
                          unit): P/G (one slab per group) automatically; 1
                          (one slab per part) may be forced.  Fused: P      */
  int32_t launches;    /* kernels one exl3_linear call enqueues (output;
                          ignored in a forced plan)                         */
  int32_t wg_cols;     /* columns per GEMM workgroup: 128, or 64 for 16-64
                          row tiles in slab mode when a layer has fewer
                          workgroups than compute units (then both halves'
                          workgroups of a 128-column block are summed by the
                          output stage); may be forced                      */
  size_t workspace;    /* bytes of workspace this plan needs: 0, or
                          EXL3_WORKSPACE_COUNTER_BYTES + the slabs, and
                          for DENSE then (256-byte aligned) K*N fp16 of
                          dequantized weights                               */
} exl3_plan;

/* ---------------------------------------------------------------- calls */

/* Input rotation (TensorFold PR, "Arithmetic" step 1; cuda-exl3 README,
 * "One op per layer", first bullet):
 *   x_rot[s][m][k] = fp16_rne( 2^-4 * H128( x[m][:] * suh[s][:] )[k] )
 * per 128-element block, for every shard s, computed in fp32 with the
 * butterfly strides 1, 2, ..., 64 in ascending order; x*suh is exact.
 *   x      [M][K] bf16 or fp16 bits (x_dtype)
 *   suh    [n_shards][K] fp16 bits
 *   x_rot  fp16 bits (output, written completely), n_shards * M * K values
 *          in K-STEP TILES: x_rot[s][k/32][m][pos(k%32)], i.e. for every
 *          shard the K/32 groups of 32 k are stored one after another, each
 *          holding all M rows (64 bytes per row), so the 32-k slice of any
 *          run of rows is one contiguous block.  Within a row's 32 values the
 *          eight 4-element chunks are stored in the order 0, 2, 1, 3, 4, 6,
 *          5, 7 (pos), so the 8 values one matrix-core lane multiplies are 16
 *          contiguous bytes.  Only the memory order differs from the formula;
 *          for M == 1 it is the row itself, chunk-permuted.
 * Errors: EXL3_ERR_INVALID_ARG for K % 128 != 0, M < 0, n_shards out of
 * range, a null or misaligned pointer, or an unknown dtype. */
exl3_status exl3_input_transform(const void *x, int32_t x_dtype, int32_t M, int32_t K,
                                 const uint16_t *suh, int32_t n_shards, uint16_t *x_rot,
                                 void *stream);

/* The input rotation of a down projection with SwiGLU folded in (cuda-exl3
 * README, "MoE throughput": SwiGLU folded into the down projection's input
 * transform).  gate_up [M][2K] in `dtype` (bf16 or fp16) is the gate_up
 * layer's output, gate = columns 0..K-1, up = K..2K-1; the value rotated is
 * what the unfused pair would store:
 *   act[m][k] = rne_dtype( silu(g) * u ),  silu(g) = g / (1 + e^-g)
 * in fp32, e^x by Cody-Waite range reduction (ln 2 split into a 12-bit head
 * and a tail) and the degree-7 Taylor polynomial of e^r, every step one IEEE
 * fp32 operation in a fixed order, then x_rot exactly as
 * exl3_input_transform(act).  Errors as exl3_input_transform. */
exl3_status exl3_input_transform_swiglu(const void *gate_up, int32_t dtype, int32_t M, int32_t K,
                                        const uint16_t *suh, int32_t n_shards, uint16_t *x_rot, void *stream);

/* Bytes of workspace exl3_linear needs for `M` rows of weight `w` (0 when
 * the plan needs none): the split-k partials and arrival counters that the
 * cuda-exl3 README ("VRAM") keeps in a process-wide workspace rather than
 * per layer.  Returns 0 and sets exl3_last_error() if `w` is invalid. */
size_t exl3_workspace_bytes(const exl3_weight *w, int32_t M);

/* The quantized linear on rotated activations (cuda-exl3 README, "One op per
 * layer"; TensorFold PR, "Arithmetic" steps 2 and 3):
 *   z[m][n] = sum_k x_rot[s(n)][m][k] * W_q[k][n]   (fp16 products, fp32 sums
 *             in P shape-fixed K parts, summed in the plan's fixed order)
 *   y[m][n] = rne_out( svh[n] * 2^-3 * H128(z[m][:])[n] )  per 128-col block
 * where s(n) is the shard holding absolute column n.
 *   x_rot     n_shards * M * K fp16 bits in the k-step tile order written by
 *             exl3_input_transform
 *   y         [M][N] in y_dtype (output, written completely)
 *   workspace at least exl3_workspace_bytes(w, M) bytes (may be NULL if 0).
 *             Its first EXL3_WORKSPACE_COUNTER_BYTES are arrival counters that
 *             must be zero on entry (allocate the workspace zeroed once) and
 *             are zero again when the call's kernels end; the rest may hold
 *             anything.  A workspace serves one call at a time.
 * In slab mode the workgroups of a tile that finish first store their
 * partial and count their arrival; the last to arrive sums the partials in
 * the plan's order and writes y (TensorFold PR, "Arithmetic": the last part
 * to finish adds the parts in part order).  No workgroup waits for another.
 * Errors: EXL3_ERR_INVALID_ARG for a bad weight view (see exl3_weight),
 * pointer or dtype; EXL3_ERR_WORKSPACE if the workspace is too small;
 * EXL3_ERR_LAUNCH if HIP refuses a launch. */
exl3_status exl3_linear(const exl3_weight *w, const uint16_t *x_rot, int32_t M, void *y,
                        int32_t y_dtype, void *workspace, size_t workspace_bytes, void *stream);

/* The plan exl3_linear would use for M rows (HOST output), and the one
 * exl3_linear_ex would use with `force` (HOST, may be NULL).  The plan's
 * workspace is the process-wide scratch of the cuda-exl3 README ("VRAM":
 * activation and split-k workspaces are process-wide, not per layer); its
 * shape-fixed parts are the TensorFold PR's ("Arithmetic").  Errors as
 * exl3_linear_ex's plan checks (the call names the failed check). */
exl3_status exl3_plan_query(const exl3_weight *w, int32_t M, exl3_plan *plan);
exl3_status exl3_plan_query_ex(const exl3_weight *w, int32_t M, const exl3_plan *force, exl3_plan *plan);

/* exl3_linear with parts of the plan forced (HOST `force`; a field <= 0, or
 * EXL3_MODE_AUTO / EXL3_DECODER_AUTO, keeps the automatic choice).  Forcing
 * `mode`, `bm`, `decoder` or `unit` never changes the output bits; forcing
 * `parts` (with `groups`, else G = P) changes the K summation tree and
 * therefore the bits (for tests and measurement).  `groups` may only be
 * forced together with `parts`; mode FUSED with G > 1 groups of several parts
 * is EXL3_ERR_UNSUPPORTED (the fused fold has one level). */
exl3_status exl3_linear_ex(const exl3_weight *w, const uint16_t *x_rot, int32_t M, void *y,
                           int32_t y_dtype, void *workspace, size_t workspace_bytes, void *stream,
                           const exl3_plan *force);

/* exl3_linear for callers that cannot allocate (code under graph capture,
 * serving loops and harnesses that forbid hipMalloc): no workspace
 * argument.  The split-k partials and arrival counters live in a device
 * array of EXL3_NOALLOC_SCRATCH_BYTES that the library owns, one per GPU it
 * runs on, held until the process ends.  The output has exactly the bits of
 * exl3_linear (the same part tree): the planner's schedule when its
 * workspace fits the array, else another schedule of the same tree that
 * fits (no dequantized weights, row chunks of the partials, the one-level
 * fused fold, or smaller row tiles).  The call allocates and frees nothing
 * and calls no allocating routine; it is asynchronous on `stream`.  All
 * calls on one GPU share that GPU's array and it keeps the last call's
 * contents (the counters are left zero): calls that overlap on one GPU race.
 * Errors as exl3_linear, and EXL3_ERR_UNSUPPORTED (naming the sizes) if no
 * schedule of the layer's tree fits the array. */
#define EXL3_NOALLOC_SCRATCH_BYTES (64u << 20)
exl3_status exl3_linear_noalloc(const exl3_weight *w, const uint16_t *x_rot, int32_t M, void *y, int32_t y_dtype,
                                void *stream);

/* Workspace bytes for exl3_linear_ex with the same `force`. */
size_t exl3_workspace_bytes_ex(const exl3_weight *w, int32_t M, const exl3_plan *force);

/* The whole layer in one call, from x instead of x_rot:
 *   y = exl3_linear(w, exl3_input_transform(x, w->suh))
 * with exactly those bits.  x is [M][K] in x_dtype (EXL3_BF16 or EXL3_F16),
 * y [M][N] in y_dtype; `w` needs trellis and suh.  The cuda-exl3 README
 * ("Two further departures") keeps the transform a separate kernel, where
 * upstream fuses it into the GEMM behind a grid-wide sync; this entry point
 * keeps both calls available and adds a third way for the plans whose GEMM
 * is the small-tile kernel (16-64 row tiles), whose workgroups' K ranges
 * fit their LDS stage slots, and whose tile rows times stages per quad is
 * at most 16: every workgroup rotates its own rows and K range of x
 * straight into LDS (the same fp32 arithmetic, rounded once to fp16), so
 * the call is one launch with no x_rot in memory and no workgroup waits
 * for another.  Since every workgroup of a row tile repeats that work, the
 * last bound keeps it shorter than the launch it saves.  Other plans run
 * the transform into the workspace, then the GEMM (two launches, as the
 * separate calls would).
 *   workspace at least exl3_forward_workspace_bytes(w, M) bytes: the plan's
 *             own workspace (arrival counters first, zero on entry as for
 *             exl3_linear), plus room for x_rot when the rotation does not
 *             run in the GEMM.  x_rot then starts after both the plan's
 *             workspace and the first EXL3_WORKSPACE_COUNTER_BYTES, so the
 *             counters keep their zeros for the next call that shares the
 *             workspace.
 * Uses the tuned schedule of the shape and M bucket when one is set (see
 * exl3_tune).  Errors as exl3_linear, and EXL3_ERR_INVALID_ARG for a bad
 * x pointer or x_dtype. */
exl3_status exl3_forward(const exl3_weight *w, const void *x, int32_t x_dtype, int32_t M, void *y, int32_t y_dtype,
                         void *workspace, size_t workspace_bytes, void *stream);
size_t exl3_forward_workspace_bytes(const exl3_weight *w, int32_t M);

/* ------------------------------------------------ schedule autotuner
 * (cuda-exl3 README, "Where the time goes": the best tile tier depends on
 * the shape, not only the batch, so the tiers are timed once per distinct
 * shape and the winner cached; tuning is skipped under graph capture, where
 * the planner's cost model is the fallback.)  Every candidate is a schedule
 * of the shape's own part tree (decoder, rows per tile, mode, unit,
 * workgroup width), so tuning never changes an output bit.  The table is
 * process-wide, keyed by (K, N, bits, codebook, shard widths, M bucket =
 * the next power of two >= M); exl3_linear, exl3_workspace_bytes and
 * exl3_plan_query use a tuned schedule when no plan is forced and it is
 * valid at their M, else the planner's.  Tune before sizing workspaces: a
 * tuned schedule may need more workspace than the planner's.
 *
 * exl3_tune runs every candidate that fits `workspace` once untimed and
 * `reps` times between two events on `stream` (it synchronizes the
 * stream), writing y each time, and records the fastest (the planner's
 * unless beaten by more than 2%); *best (HOST, may be NULL) receives it.
 * `ws` (HOST) holds n_w views of the same shape, e.g. copies of one weight
 * whose trellises together exceed the caches: the timed calls cycle
 * through them, so the timing sees weights streamed from HBM as a model's
 * layers are (one view times a warm, cache-resident weight).
 * EXL3_ERR_INVALID_ARG if a view differs in shape; EXL3_ERR_UNSUPPORTED
 * while the stream is being captured; EXL3_ERR_WORKSPACE if no candidate
 * fits. */
exl3_status exl3_tune(const exl3_weight *ws, int32_t n_w, const uint16_t *x_rot, int32_t M, void *y,
                      int32_t y_dtype, void *workspace, size_t workspace_bytes, int32_t reps, void *stream,
                      exl3_plan *best);

/* Workspace that fits every candidate exl3_tune tries for M rows. */
size_t exl3_tune_workspace_bytes(const exl3_weight *w, int32_t M);

/* Record a schedule for (shape, M bucket) as exl3_tune would (e.g. one
 * tuned earlier and saved): validated like a forced plan; its parts and
 * groups must be the shape's own (EXL3_ERR_INVALID_ARG otherwise). */
exl3_status exl3_tune_set(const exl3_weight *w, int32_t M, const exl3_plan *plan);

/* Forget every tuned schedule. */
void exl3_tune_clear(void);

/* Human-readable status name, and the thread's last error message.  Calls
 * refuse what they cannot run rather than misread it (TensorFold PR, "What
 * it adds": a weight is refused when its format is not loaded) and the
 * message says which check failed and by how much (cuda-exl3 README,
 * "Loading into a dim vLLM has padded"). */
const char *exl3_status_str(exl3_status s);
const char *exl3_last_error(void);
int32_t exl3_abi_version(void);

/* ------------------------------------------- test and measurement hooks */

/* Every state of one codebook through the device decoder:
 * out[s] = fp16 bits of codebook(s), s = 0..65535 (cuda-exl3 README, "What
 * is supported"; TensorFold PR, "Tests (GB10)" first bullet). */
exl3_status exl3_debug_codebook(int32_t codebook, uint16_t *out, void *stream);

/* The whole W_q [K][N] (fp16 bits) decoded by the GEMM's own staging and
 * unpacking path (TensorFold PR, "Tests (GB10)" second bullet). */
exl3_status exl3_debug_decode(const exl3_weight *w, uint16_t *wq, void *stream);

/* The dense decoder's first stage alone: the whole W_q decoded once into
 * matrix-core B fragments, the layout exl3_linear's dense decoder keeps in
 * its workspace (TensorFold PR, "Tests (GB10)" second bullet: the decoded
 * weights checked against the reference's).  frags (device, frag_bytes >=
 * K*N*2) receives [K/32][N/128][8][64][8] fp16 bits: for the 32-k step ks,
 * the 128-column block nb, fragment f = 2w + h and lane L = 16g + j, the 8
 * values are W_q[32ks + k][128nb + c], c = 16(2w + j/8) + j%8 + 8h, at the 8
 * k of the rotated activations' 16-byte piece g (4-element chunks c(2g) and
 * c(2g+1), c = 0, 2, 1, 3, 4, 6, 5, 7), so a lane's B values meet its A
 * values in one matrix-core product.  EXL3_ERR_WORKSPACE if frag_bytes is
 * short. */
exl3_status exl3_debug_dequant(const exl3_weight *w, uint16_t *frags, size_t frag_bytes, void *stream);

/* The dense decoder's second stage alone, over fragments that
 * exl3_debug_dequant wrote (device, frag_bytes >= K*N*2), for timing its
 * two launches apart.  The dense GEMM runs 256 x 256 workgroup tiles over
 * whole rounds of the GPU's CUs and the column blocks after them as
 * 256 x 128 tiles, twice as many workgroups of half the work (columns only
 * split, so the bits are the same; see the plan's `launches`).  which: 1
 * the 256 x 256 launch, 2 the 256 x 128 launch, 3 both (y then equals
 * exl3_linear's with the dense decoder).  *bulk_blocks (HOST, may be NULL)
 * receives the column blocks of the 256 x 256 launch (N/128 when nothing
 * is split).  The plan is exl3_linear's with the dense decoder forced; it
 * must be one part per workgroup, fused, in one row chunk, else
 * EXL3_ERR_UNSUPPORTED.  Needs no workspace. */
exl3_status exl3_debug_dense_gemm(const exl3_weight *w, const uint16_t *frags, size_t frag_bytes,
                                  const uint16_t *x_rot, int32_t M, void *y, int32_t y_dtype, int32_t which,
                                  int32_t *bulk_blocks, void *stream);

/* The trellis GEMM stage alone, the kernel slab mode runs before the
 * output stage: the fp32 sum of every K part (unit 1, the default), or of
 * every group (force->unit = P/G, the automatic slab plan's own stage),
 *   z_parts[u][m/4][n][m%4] = sum_{k in unit u} x~[s(n)][m][k] * W_q[k][n]
 * with the parts of a unit added in part order (TensorFold PR, "Arithmetic"
 * step 2, with the ordered K parts of the cuda-exl3 README's split-k, "Two
 * further departures").  The plan is the one exl3_linear would use, or
 * `force` (HOST, may be NULL) as in exl3_linear_ex, with the mode set to
 * slabs; x_rot as for exl3_linear.  z_parts (device) needs
 * (P/unit) * ceil(M/4) * 4 * N * 4 bytes (z_bytes, checked;
 * EXL3_ERR_WORKSPACE if short); rows past M in the last group of four hold
 * unspecified finite values.  Exactly what exl3_debug_epilogue reads. */
exl3_status exl3_debug_parts(const exl3_weight *w, const uint16_t *x_rot, int32_t M, float *z_parts,
                             size_t z_bytes, void *stream, const exl3_plan *force);

/* The output stage alone, the stage slab mode runs after the GEMM:
 * y = rne_out(svh * 2^-3 * H128(z)) with z the fp32 sum of the n_parts slabs
 * in `groups` groups of n_parts/groups consecutive slabs: each group added in
 * slab order (first copied), then the groups in order (first copied); with
 * groups == n_parts, z = ((z_parts[0] + z_parts[1]) + ...) (TensorFold PR,
 * "Arithmetic" step 3 and the ordered part sum).  z_parts is in the
 * partial-slab layout [n_parts][ceil(M/4)][N][4] fp32: element (part, m, n)
 * at ((part * ceil(M/4) + m/4) * N + n) * 4 + m%4.  EXL3_ERR_INVALID_ARG if
 * groups does not divide n_parts. */
exl3_status exl3_debug_epilogue(const float *z_parts, int32_t n_parts, int32_t groups, int32_t M,
                                const exl3_weight *w, void *y, int32_t y_dtype, void *stream);

/* ---------------------------------------------- mixture of experts
 * Routed experts as one grouped GEMM (cuda-exl3 README, "What is
 * supported": the (token, expert) pairs are sorted by expert and each
 * expert's run is padded to whole row blocks, so every block belongs to one
 * expert and the GEMM offsets the trellis by the block's expert; blocks of
 * no expert are skipped; "Determinism": routed rows are written and each
 * token's top-k rows summed in a fixed order in fp32, rounded once).  Each
 * routed row has exactly the bits exl3_linear gives that token on its
 * expert's weight alone (the part tree is the expert shape's own).
 *
 * Pair p = t * topk + j is token t's j-th expert.  The routed buffers have
 * exl3_moe_rows_max(T, topk, E, block) rows: at most T*topk pairs plus the
 * padding of every expert with pairs, in whole blocks (0 if that exceeds
 * the supported rows). */
int32_t exl3_moe_rows_max(int32_t T, int32_t topk, int32_t E, int32_t block);

/* topk_ids [T][topk] int32 (device; ids outside 0..E-1 drop their pair) ->
 *   row_pair     [rows]          pair of each routed row, -1 for padding
 *   block_expert [rows / block]  expert of each row block, -1 after the last
 *   pair_row     [T * topk]      routed row of each pair, -1 if dropped
 * Expert e's pairs occupy rows start(e) .. start(e) + count(e) - 1, start(e)
 * the whole-block padded counts of the experts before it; within that run
 * the order of the pairs may vary between runs (every result is the same).
 * block 16, 32 or 64; E <= 4096; topk <= 64.  One workgroup. */
exl3_status exl3_moe_align(const int32_t *topk_ids, int32_t T, int32_t topk, int32_t E, int32_t block,
                           int32_t *row_pair, int32_t *block_expert, int32_t *pair_row, void *stream);

/* The input rotation of every routed row: row r rotates token row_pair[r] /
 * topk of x ([T][K], or with `swiglu` the gate_up output [T][2K] as in
 * exl3_input_transform_swiglu) with the suh rows of its block's expert,
 * suh [E][n_shards][K] fp16; padding rows rotate zeros.  x_rot as from
 * exl3_input_transform for `rows` rows (rows = exl3_moe_rows_max). */
exl3_status exl3_moe_input_transform(const void *x, int32_t x_dtype, int32_t swiglu, int32_t T, int32_t K,
                                     const uint16_t *suh, int32_t n_shards, int32_t E, const int32_t *row_pair,
                                     const int32_t *block_expert, int32_t topk, int32_t block, int32_t rows,
                                     uint16_t *x_rot, void *stream);

/* Workspace for exl3_moe_linear (same validity rules as exl3_workspace_bytes). */
size_t exl3_moe_workspace_bytes(const exl3_weight *w, int32_t rows, int32_t block);

/* The grouped GEMM: `w` describes expert 0 and the E experts are stacked
 * behind it at fixed strides: trellis [E][K/16][N/16][16*bits], suh
 * [E][n_shards][K], svh [E][N], bias [E][N] (if any).  Row block b of x_rot
 * (rows = a multiple of `block`) is multiplied by expert block_expert[b]'s
 * weight (skipped when -1) into y [rows][N]; rows of padding hold
 * unspecified values.  The ALU tiles of `block` rows with the output stage
 * in the GEMM.  Errors as exl3_linear; EXL3_ERR_UNSUPPORTED if the rows
 * need more finishing counters than the workspace holds and the tree has no
 * fused schedule. */
exl3_status exl3_moe_linear(const exl3_weight *w, int32_t E, const uint16_t *x_rot, int32_t rows,
                            const int32_t *block_expert, int32_t block, void *y, int32_t y_dtype, void *workspace,
                            size_t workspace_bytes, void *stream);

/* exl3_moe_linear with the decoder chosen by the caller: EXL3_DECODER_AUTO
 * (what exl3_moe_linear does), EXL3_DECODER_ALU (the ALU tiles above), or
 * EXL3_DECODER_TABLE: one persistent workgroup per CU decodes part of every
 * weight through a 65,536-entry table in LDS (as exl3_linear's table
 * decoder), each (16-row block, 128-column block) one fused unit that folds
 * the shape's part tree in two levels (the parts of each group in order,
 * then the groups in order, the first term copied each time), so each routed
 * row still has exl3_linear's bits; it needs no workspace.  AUTO takes the
 * table when block is 16, the stacked trellis is at most 2 GiB and there
 * are at least 256 such units (enough to fill the GPU without splitting K;
 * cuda-exl3 README, "What is supported": decode-bound expert GEMMs at a
 * handful of rows per expert).  EXL3_ERR_UNSUPPORTED for TABLE with another
 * block or a larger stack; EXL3_ERR_INVALID_ARG for another decoder. */
exl3_status exl3_moe_linear_ex(const exl3_weight *w, int32_t E, const uint16_t *x_rot, int32_t rows,
                               const int32_t *block_expert, int32_t block, void *y, int32_t y_dtype, void *workspace,
                               size_t workspace_bytes, void *stream, int32_t decoder);

/* out[t][n] = rne_dtype( sum over j of topk_weights[t][j] * y_routed[pair_row[t*topk+j]][n] ),
 * the sum in fp32 from 0 in j order, each product rounded to fp32 before it
 * is added; dropped pairs add nothing.  y_routed [rows][N] and out [T][N] in
 * `dtype`; topk_weights fp32 [T][topk]; N even. */
exl3_status exl3_moe_combine(const void *y_routed, int32_t dtype, const int32_t *pair_row, const float *topk_weights,
                             int32_t T, int32_t topk, int32_t N, void *out, void *stream);

/* ------------------------------------------------- measurement rulers
 * Not part of the layer API: simple kernels that measure, in the same run
 * as the layer timings, what this GPU's HBM, matrix cores and decode path
 * deliver, so the layer figures can be read against attainable rates as
 * well as the data-sheet peaks (cuda-exl3 README, "Measured": a matmul
 * reads k*n*bits/8 bytes and does 2*m*k*n flops, speed of light is the max
 * of the two limits, and the roofline there is itself measured).  Each writes EXL3_RULER_WORDS words (or one word
 * per weight block) to a caller-owned device buffer and is asynchronous on
 * `stream`. */
#define EXL3_RULER_WORDS 262144

/* Streaming read of buf[0 .. bytes): EXL3_RULER_WORDS threads each XOR the
 * 4-byte words of their grid-stride share of the 16-byte words into
 * out[t], so the XOR of all out words is the XOR of the whole buffer.
 * EXL3_ERR_INVALID_ARG unless bytes is a positive multiple of 16 and buf and
 * out are 16-byte aligned. */
exl3_status exl3_debug_stream_read(const void *buf, size_t bytes, uint32_t *out, void *stream);

/* Matrix-core loop: EXL3_RULER_WORDS / 64 waves each run `iters` rounds of
 * 16 independent v_mfma_f32_16x16x32_f16 chains with every A and B element
 * the fp16 value `one` (bits); out[t] (float) = the sum of the lane's 16
 * chains' first elements = 512 * iters * one^2 while exact.  Work:
 * 16384 * 16 * iters * EXL3_RULER_WORDS / 64 flops.  iters in 1 .. 2^20.
 * With one = 0 the operands are instead two sets of pseudo-random fp16
 * values (magnitudes in [0.5, 1), random signs, from a hash of the thread
 * index) used alternately, so every product's inputs differ from the last
 * one's, as on real data (constant operands let the chip hold a higher
 * clock); then |out[t]| <= 512 * iters and every word is finite. */
exl3_status exl3_debug_mfma_loop(int32_t iters, uint16_t one, float *out, void *stream);

/* Decode ruler: every weight of `w` staged and decoded as the GEMM kernels
 * do, with no matrix products and no weight stores.  out[kb * (N/128) + nb]
 * (uint32, (K/128) * (N/128) words) = XOR of block (kb, nb)'s decoded fp16
 * values at even k in the low 16 bits and at odd k in the high 16 bits. */
exl3_status exl3_debug_decode_rate(const exl3_weight *w, uint32_t *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* EXL3_H */
