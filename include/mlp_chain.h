/*
 * mlp_chain.h -- C ABI of the tile-synchronized MLP GEMM chain for MI355X (gfx950).
 *
 * The operation is the transformer MLP as a chain of two dependent GEMMs:
 *
 *     T = act(X * W1)      (first GEMM, activation fused into its epilogue)
 *     Y = T * W2           (second GEMM, consumes T)
 *
 * which the CuSync README (github.com/microsoft/cusync, opening paragraph)
 * describes as a producer kernel and a consumer kernel whose dependent tiles
 * (thread blocks) are synchronized by policies instead of whole-kernel
 * ordering, so that independent tiles run concurrently and fill the last
 * wave of thread blocks; the same README's paragraph on the GPT-3 / LLaMA MLP
 * graphs fuses GeLU into the first GeMM.  The policies here are:
 *
 *   MLP_POLICY_STREAM_ORDERED  two kernels on one stream (GEMM1+act, then
 *                              GEMM2): kernel-level dependency, the baseline.
 *   MLP_POLICY_ROW_SYNC        one persistent kernel; a GEMM2 tile waits until
 *                              every GEMM1 tile of its row block is done.
 *   MLP_POLICY_TILE_SYNC       one persistent kernel; a GEMM2 tile waits, K
 *                              chunk by K chunk, only for the GEMM1 tile that
 *                              produced that chunk.
 *
 * All three compute bit-identical outputs: they share the K split and the
 * accumulation order of every output element (each may use its own tile
 * shape, which changes no element's arithmetic); they differ only in when
 * tiles run.
 *
 * Numerics: inputs and outputs are fp16 or bf16; products accumulate in fp32
 * on the matrix cores; the activation is applied to the fp32 accumulator(s);
 * T is rounded to the storage dtype once (round to nearest even), then the
 * second GEMM accumulates in fp32 and rounds Y the same way.
 *
 * Layouts (all row-major, contiguous, same dtype, 16-byte aligned base):
 *   x   [M, H]
 *   w1  [H, I]      for gelu_tanh / none
 *       [H, 2I]     for swiglu: gate = w1[:, 0:I], up = w1[:, I:2I]
 *   w2  [I, H]
 *   out [M, H]
 * H and I must be multiples of 8 (16-byte rows); M is any value >= 1.
 *
 * Activations:
 *   none       a = h
 *   gelu_tanh  a = 0.5 h (1 + tanh(sqrt(2/pi) (h + 0.044715 h^3)))
 *   swiglu     a = silu(g) * u,  silu(g) = g / (1 + exp(-g))
 *
 * Pointers: x, w1, w2 and out are DEVICE pointers owned by the caller.  The
 * stream argument is a hipStream_t passed as void* (NULL = default stream).
 * The handle owns a device workspace (the intermediate T [M, I], stored
 * with its rows padded to a multiple of 64 elements so that every 128-byte
 * line of it lies in one row, per-tile
 * ready flags, per-row-block counters, two sets of per-XCD tile-queue
 * counters, a status word, and for split tiles fp32 partials, per-tile
 * arrival counters and per-part ready words), allocated by create and freed
 * by destroy.
 *
 * Concurrency: runs on one handle must be ordered on one stream (they share
 * the workspace); separate handles are independent.  All entry points are
 * thread-safe with respect to different handles.
 *
 * Errors: functions return MLP_OK (0) or a negative code; the message of the
 * last failure on the calling thread is available from mlp_chain_last_error.
 */
#ifndef MLP_CHAIN_H
#define MLP_CHAIN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct mlp_chain* mlp_chain_t;

enum { MLP_ACT_NONE = 0, MLP_ACT_GELU_TANH = 1, MLP_ACT_SWIGLU = 2 };
enum { MLP_DTYPE_F16 = 0, MLP_DTYPE_BF16 = 1 };
enum { MLP_POLICY_STREAM_ORDERED = 0, MLP_POLICY_ROW_SYNC = 1, MLP_POLICY_TILE_SYNC = 2 };
enum { MLP_OK = 0, MLP_EINVAL = -1, MLP_ENOMEM = -2, MLP_EHIP = -3, MLP_ETIMEOUT = -4 };

/* Create a chain for fixed sizes on the current HIP device.
 * M >= 1, H >= 8 and I >= 8 with H % 8 == 0 and I % 8 == 0; act, dtype and
 * policy from the enums above.  Picks the tile configuration, allocates and
 * zeroes the workspace.  Returns NULL on error (bad argument, out of device
 * memory, HIP failure) with mlp_chain_last_error() set.
 * (CuSync README, opening paragraph: policies over a producer/consumer chain.) */
mlp_chain_t mlp_chain_create(int64_t M, int64_t H, int64_t I, int act, int dtype, int policy);

/* Enqueue one chain pass Y = act(X W1) W2 on `hip_stream` with the handle's
 * policy.  Asynchronous: never synchronizes the host.  Returns MLP_EINVAL for
 * a NULL handle or a NULL / non-16-byte-aligned pointer, MLP_EHIP if a launch
 * fails.  A consumer tile that waits longer than the spin limit for its
 * producer gives up and records MLP_ETIMEOUT in the handle's status word
 * (see mlp_chain_status); its output is then undefined.
 * A run's launches depend on nothing the host changes between runs (the
 * fused policies keep the epoch of their ready flags on the device), so
 * they may be captured into a HIP graph and replayed, every policy (the
 * same pointers each replay; replays and direct runs of one handle on one
 * stream may be mixed).
 * The fused policies' persistent kernel sizes its grid to what the GPU holds
 * at once and its waits end only once every workgroup is running: a kernel
 * of another stream that keeps CUs occupied meanwhile can hold consumers in
 * their waits until the watchdog gives up (MLP_ETIMEOUT, output undefined).
 * Run the fused policies without concurrent kernels on the same GPU, or use
 * stream_ordered there.
 * (CuSync README, opening and MLP paragraphs.) */
int mlp_chain_run(mlp_chain_t h, const void* x, const void* w1, const void* w2, void* out,
                  void* hip_stream);

/* Row strides (in elements) of the weights the handle's runs read: W1
 * [H, g I] with rows ldw1 >= g I apart, W2 [I, H] with rows ldw2 >= H apart
 * (g = 2 for SwiGLU, else 1; gate columns 0..I-1 and up columns I..2I-1 of a
 * W1 row stay where mlp_chain_run describes them; the padding between rows
 * is never read).  Both multiples of 8 and at most 2^24.  The default is
 * dense rows (g I and H).  Applies to every later run of the handle, one
 * layer or several (every layer's weights have these strides).  Returns
 * MLP_EINVAL for a NULL handle or a stride outside those bounds.
 * (No page defines a weight layout: this is a deployment choice the library
 * offers because rows that are a whole number of kilobytes apart put every
 * row of a column panel on the same class of 128-byte lines, which streams
 * slower; see mlp_chain_weight_ld.) */
int mlp_chain_set_weight_ld(mlp_chain_t h, int64_t ldw1, int64_t ldw2);

/* The weight row strides this library streams fastest for these sizes: the
 * smallest ldw1 >= g I and ldw2 >= H that are an odd number of 128-byte
 * lines (64 mod 128 elements), so that consecutive rows of a column panel
 * cycle through all eight classes of lines.  Host-only; returns MLP_EINVAL
 * for NULL outputs or sizes mlp_chain_create would reject. */
int mlp_chain_weight_ld(int64_t H, int64_t I, int act, int64_t* ldw1, int64_t* ldw2);

/* A chain of `layers` MLP layers (1..8), 2 x layers dependent GEMMs:
 * layer l computes Y_l = act(Y_{l-1} W1_l) W2_l, with Y_{-1} = x and the last
 * layer's Y written to out; every layer has the sizes of mlp_chain_create
 * (H wide in and out, I inner), the same activation and dtype, and its own
 * weights.  With the fused policies all 2 x layers GEMMs run in ONE
 * persistent kernel: a layer's GEMM2 tiles wait for the GEMM1 tiles of its
 * intermediate they read, and the next layer's GEMM1 tiles wait, K chunk by
 * K chunk, for the GEMM2 tiles of Y_l they read, so one layer's consumers
 * overlap the previous layer's tail -- the cross-layer overlap of the
 * megakernel discussion (Hacker News thread on megakernels vs CUDA graphs:
 * CUDA graphs do not overlap work across layers; fine-grained tasks spread
 * over the SMs).  stream_ordered launches the 2 x layers kernels in order on
 * the stream.  Every policy computes every layer with the plan
 * mlp_chain_create makes for these sizes, so outputs are bit-identical to
 * `layers` one-layer runs in sequence.  The workspace keeps every layer's
 * intermediate and every layer output but the last (rows padded to 64
 * elements).  Returns NULL on error as mlp_chain_create. */
mlp_chain_t mlp_chain_create_layers(int64_t M, int64_t H, int64_t I, int act, int dtype, int policy, int layers);

/* Enqueue one pass of a multi-layer chain: `w1` and `w2` are HOST arrays of
 * `layers` device pointers (layer l's [H, g I] and [I, H] weights, layouts
 * as for mlp_chain_run); x and out as for mlp_chain_run.  A one-layer handle
 * runs as mlp_chain_run(w1[0], w2[0]); mlp_chain_run refuses a handle of
 * more than one layer.  Errors, asynchrony and the watchdog as
 * mlp_chain_run. */
int mlp_chain_run_layers(mlp_chain_t h, const void* x, const void* const* w1, const void* const* w2, void* out,
                         void* hip_stream);

/* Release the handle and its workspace.  Waits first for the stream of the
 * handle's last run (that stream must still exist; other streams are not
 * waited for).  NULL-safe; returns MLP_OK, or MLP_EHIP if the wait or the
 * free failed.  (No page defines handle lifetime: create / run / destroy
 * with policy in {stream_ordered, row_sync, tile_sync} is the interface the
 * task statement fixes for this library.) */
int mlp_chain_destroy(mlp_chain_t h);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): one chain
 * pass Y = act(X W1) W2 like mlp_chain_create + mlp_chain_run + destroy,
 * with the same plan (so the same output bits as mlp_chain_run), but with
 * no handle and no allocation: the workspace lives in a static device
 * scratch of 128 MiB that the library holds on each device it runs on from
 * the first call there until the process ends.  The first call on a device
 * looks the scratch up (make it outside any graph capture); later calls
 * call no allocating routine.  Each call first clears the scratch's
 * synchronization words with a small kernel on `hip_stream` (no memset), so
 * it does not depend on what an earlier call left there.  Calls that
 * overlap on one device race on the scratch and must be ordered (one
 * stream, or events).  Arguments as mlp_chain_create and mlp_chain_run;
 * `status` is NULL or a 4-byte aligned device uint32 owned by the caller:
 * it is zeroed when the pass starts and nonzero after it if a consumer tile
 * gave up waiting (output then undefined).  Asynchronous.  Returns
 * MLP_EINVAL for bad sizes, enums or pointers, or when the plan's
 * workspace exceeds the scratch (the message gives both sizes; the
 * 8192^3 chain's intermediate alone fills it), MLP_EHIP if the scratch
 * lookup or a launch fails. */
int mlp_chain_run_noalloc(int64_t M, int64_t H, int64_t I, int act, int dtype, int policy, const void* x,
                          const void* w1, const void* w2, void* out, void* status, void* hip_stream);

/* Enqueue one phase alone, with the same kernels and tiles as the
 * stream-ordered policy: phase 1 = GEMM1 + activation, writing the handle's
 * intermediate T; phase 2 = GEMM2, reading the handle's T and writing out.
 * Unused pointers may be NULL (phase 1 ignores w2/out, phase 2 ignores x/w1).
 * It times the best unsplit GEMMs for an overhead figure in the style of the
 * FLUX summary card's Effective Communication Time (Interesting ideas, I2:
 * total time minus the best unsplit GEMM time).  Returns as mlp_chain_run,
 * and MLP_EINVAL for a phase other than 1 or 2. */
int mlp_chain_run_phase(mlp_chain_t h, int phase, const void* x, const void* w1, const void* w2,
                        void* out, void* hip_stream);

/* Read the sticky device status after the handle's work: the status word
 * is copied on the stream of the handle's last run, which is then
 * synchronized (that stream must still exist; other streams of the process
 * are not waited for).  Returns MLP_OK, or MLP_ETIMEOUT if a consumer tile
 * gave up waiting since the last call.  Reading an error also clears it and
 * re-zeroes the handle's flags and counters (a device-wide synchronization,
 * on this recovery path only) so that the next run starts clean.  Returns
 * MLP_EINVAL for a NULL handle and MLP_EHIP if the device reports an error.
 * (The pages give no failure model; the watchdog and this status word are
 * this library's own, as the benchmark spec's error contract asks.) */
int mlp_chain_status(mlp_chain_t h);

/* Message describing the last failed call on this thread ("" if none).  The
 * string is owned by the library and valid until the next call on the thread.
 * (Part of the error contract the benchmark spec fixes; no page defines it.) */
const char* mlp_chain_last_error(void);

/* Plan and launch facts of a handle, for tests and measurement; fills the
 * first min(n, 21) of
 *   { BM, BN1, BN2, BK, Mt, N1t, N2t, T1, T2, persistent grid,
 *     workgroups per CU, threads per workgroup, CUs, epoch,
 *     config id, workspace bytes, S1, S2, K slabs per GEMM1 part,
 *     K slabs per GEMM2 part, layers }.
 * (S1, S2: the deterministic K split of GEMM1 / GEMM2 tiles, 1 = none;
 * epoch: that of the last finished fused run, read from the device after
 * waiting for the stream of the handle's last run.)
 * Returns MLP_EINVAL for a NULL handle or array, or n < 16, MLP_EHIP if
 * reading the epoch fails. */
int mlp_chain_info(mlp_chain_t h, int64_t* info, int n);

/* The plan mlp_chain_create would make for these sizes on a GPU with `cus`
 * compute units, computed on the host alone (no device is touched): fills
 * the first min(n, 14) of
 *   { config id, S1, S2, BM, BN1, BN2, Mt, N1t, N2t, T1, T2,
 *     K slabs per GEMM1 part, K slabs per GEMM2 part,
 *     1 if the plan comes from the tuned table, else 0 }.
 * Shapes measured by the tuner (the library's table of tuned plans, for an
 * exact size and CU count; the FLUX summary card's point that kernels are
 * auto-tuned per GPU) take the measured plan; every other shape the rules.
 * A negative `cus` plans for -cus CUs with the rules alone (the tuned table
 * ignored), for tests of the rules.
 * The K split (S1, S2) depends on the sizes and `cus` only, never on the
 * policy, so all policies compute the same output bits; the tile
 * configuration may differ per policy.  The planner fills the last wave of
 * the GPU (the CuSync README, opening paragraph) by splitting K where a GEMM
 * has fewer tiles than CUs, and for the fused policies splits GEMM1 in two
 * where its tiles make between half a wave and one wave.  Returns MLP_EINVAL
 * for sizes, act or policy that mlp_chain_create would reject, |cus| < 8, a
 * NULL array or n < 3. */
int mlp_chain_plan(int64_t M, int64_t H, int64_t I, int act, int policy, int cus, int64_t* plan, int n);

/* Test hooks (never needed for normal use):
 * set the consumer spin limit (iterations of the back-off loop before a
 * consumer gives up; 0 restores the default), and make producer part
 * `tile` (ticket order: tile * S1 + part, -1 = none) skip its work and its
 * release, which forces the watchdog path without any kernel faulting or
 * hanging.
 * Return MLP_EINVAL for a NULL handle. */
int mlp_chain_debug_set_spin_limit(mlp_chain_t h, uint32_t limit);
int mlp_chain_debug_skip_producer(mlp_chain_t h, int64_t tile);

/* Force a tile configuration by id for the next runs (-1 = planner's
 * choice); used by tests and tuning sweeps.  Synchronizes the device and
 * rebuilds (and re-zeroes) the workspace; the intermediate is lost.
 * Returns MLP_EINVAL for a NULL handle or an unknown id, MLP_ENOMEM if the
 * new workspace cannot be allocated. */
int mlp_chain_debug_set_config(mlp_chain_t h, int config_id);

/* Force the number of K parts of GEMM1 tiles (s1) and GEMM2 tiles (s2), 0 =
 * planner's choice, at most 64; parts may be empty when a split exceeds the
 * K slabs.  Small-M tiles are split so that every CU streams weights; each
 * part accumulates its K range in fp32 and the last part to finish sums the
 * partials in part order, so every policy sees the same arithmetic (the
 * CuSync README names CUTLASS StreamK as the other remedy for the last
 * wave; this is a fixed, deterministic split).  Synchronizes and rebuilds
 * the workspace like mlp_chain_debug_set_config.  Returns MLP_EINVAL for a
 * NULL handle or a split outside 0..64. */
int mlp_chain_debug_set_split(mlp_chain_t h, int s1, int s2);

/* Force the number of persistent workgroups of the fused policies, 0 = the
 * planner's (as many per CU as fit, but no more than the run's whole items
 * per CU).  Values are clamped to [8, workgroups per CU x CUs]: at least one
 * workgroup per tile queue, and never more than can be resident at once
 * (the persistent kernel needs all its workgroups resident).  For
 * measurements of the schedule (the CuSync README's point about the last
 * wave of the producer kernel); takes effect on the next run.  Returns
 * MLP_EINVAL for a NULL handle or a negative value. */
int mlp_chain_debug_set_grid(mlp_chain_t h, int grid);

/* Override the order in which each XCD walks its block of the tile grid:
 * bit 0 for GEMM1, bit 1 for GEMM2, set = column-major (the tiles an XCD
 * runs together form a patch of rows x columns rather than a run along one
 * row); bits 4..7 (rx = order >> 4, one of 1, 2, 4, 8; 0 = planned) the
 * number of XCD rows of the partition of each GEMM's tile grid over the 8
 * XCDs (rx rows of 8/rx XCDs: with rx = 1 every XCD holds all row blocks,
 * so the whole GPU completes the row blocks of T one after another).  -1
 * restores the planner's choices.  The order changes which tiles share an
 * XCD's L2 at a time and, for the fused policies, when each row block of T
 * completes -- never any output value.  Takes effect on the next run.
 * Returns MLP_EINVAL for a NULL handle or a value outside those. */
int mlp_chain_debug_set_order(mlp_chain_t h, int order);

/* Test hook: put the handle's synchronization state where the fused run of
 * epoch `epoch` leaves it (every ready flag holding `epoch`, every row
 * counter at epoch x tiles per row block, modulo 2^32, both sets of queue
 * counters zero, the device's epoch word `epoch`), so that the next runs
 * use epochs epoch+1, epoch+2, ... -- e.g. across the 32-bit wrap.
 * Synchronizes the device.  Returns MLP_EINVAL for a NULL handle, MLP_EHIP
 * if the device reports an error. */
int mlp_chain_debug_set_epoch(mlp_chain_t h, uint32_t epoch);

/* Timeline trace of every policy (measurement of the non-overlapped share,
 * as the FLUX summary card advises in Interesting ideas, I3):
 * `buffer` is a DEVICE buffer of 4 * layers * (T1*S1 + T2*S2) uint64 (see
 * mlp_chain_info), NULL turns tracing off.  Each run then writes, per ticket
 * t (layer by layer, producer parts first), words 4t..4t+3 = { start, end of the part's
 * last wait (= start where nothing waits), end } on the 100 MHz realtime
 * clock, and { t | XCD << 32 |
 * HW_ID << 36 | (part wrote the tile's output) << 63 }.  The buffer stays
 * owned by the caller and must outlive the runs that use it.  Returns
 * MLP_EINVAL for a NULL handle. */
int mlp_chain_debug_set_trace(mlp_chain_t h, void* buffer);

/* Test hook: a message-passing litmus test of the hand-off between tiles
 * (the pages give no memory-ordering protocol; the CuSync README's opening
 * paragraph only says dependent tiles are synchronized).  256 workgroups run
 * `rounds` rounds in one launch; in each, every workgroup writes its share
 * of a fresh 8 KB region and publishes it exactly as a producer tile does,
 * then consumes a region one of whose two writers sits on its own XCD,
 * exactly as a consumer tile does (relaxed polls, hand-off acquire of
 * workgroup scope, or agent scope if `agent`, operand DMA into LDS), and
 * checks every word.  With `half_lines` the two writers of a region write
 * the two 64-byte halves of each of its 128-byte lines, from two XCDs.
 * DEVICE buffers, zeroed by the caller: data >= rounds MiB (256-byte
 * aligned), flags >= rounds x 1 KiB, result >= 8 uint32:
 *   result[0] = words read wrong, result[1..5] = the first one's round + 1,
 *   consumer workgroup, 16-byte chunk, word read, word expected,
 *   result[6] != 0 if a wait exceeded `spin_limit` polls (0 = default).
 * Enqueued on hip_stream.  Returns MLP_EINVAL for bad pointers or sizes
 * (rounds 1..4096), MLP_EHIP if the launch fails. */
int mlp_chain_debug_litmus(void* data, size_t data_bytes, void* flags, size_t flag_bytes, void* result, int rounds,
                           int half_lines, int agent, uint32_t spin_limit, void* hip_stream);

/* Copy the handle's intermediate T [M, I] (as left by the last run on the
 * handle) into the caller's device buffer `dst` (M * I elements of the
 * storage dtype, rows contiguous: the workspace's row padding is dropped),
 * enqueued on `hip_stream` after the handle's work.  For
 * tests that check the intermediate itself.  Returns MLP_EINVAL for a NULL
 * handle or buffer, MLP_EHIP if the copy cannot be enqueued. */
int mlp_chain_debug_read_intermediate(mlp_chain_t h, void* dst, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* MLP_CHAIN_H */
