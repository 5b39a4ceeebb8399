/*
 * mk.h — C ABI of the MI355X (gfx950) decode library.
 *
 * One greedy decode step of a Llama-style decoder runs as ONE persistent
 * kernel launch (mk_decode_step), or, for A/B comparison, as one launch per
 * fused op and layer (mk_decode_step_multikernel).  The step is the fused op
 * sequence that the page "Megakernels: Deleting the Kernel Boundary to Win
 * Back Microseconds" lists in its section "One launch, one interpreter"
 * (RMSNorm+QKV+RoPE, attention, attention reduce, O-proj+residual,
 * RMSNorm+up/gate+SiLU, down-proj+residual, RMSNorm+LM head), executed by an
 * on-device interpreter over per-CU instruction queues built on the host ahead
 * of time (same section), with the data dependencies that the kernel boundary
 * used to give rebuilt on device (section "Correctness without the free
 * barrier").
 *
 * Conventions for every entry point:
 *   - Return 0 (MK_OK) or a negative mk_status; no C++ exception crosses the ABI.
 *   - "device pointer" arguments are HIP device allocations on the handle's
 *     device; "host pointer" arguments are ordinary CPU memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *   - The caller owns every buffer it passes; the library owns the handle and
 *     everything it allocates.
 */
#ifndef MK_H
#define MK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MK_OK = 0,
    MK_ERR_INVALID_ARG = -1,       /* null pointer, out-of-range value */
    MK_ERR_UNSUPPORTED_SHAPE = -2, /* config the kernels do not handle */
    MK_ERR_HIP = -3,               /* a HIP runtime call failed; see mk_last_error */
    MK_ERR_OOM = -4,               /* device or host allocation failed */
    MK_ERR_STATE = -5,             /* call order violated (e.g. decode before load) */
    MK_ERR_DEVICE = -6             /* the kernel reported an error record */
} mk_status;

/* Model and run shape.  Llama-style decoder: per layer RMSNorm, Q/K/V, RoPE
 * (rotate-half pairs (i, i + D/2), frequency theta^(-2i/D)), causal GQA
 * attention (query head h reads KV group h * n_kv_heads / n_q_heads), O-proj
 * + residual, RMSNorm, SwiGLU MLP, down-proj + residual; then RMSNorm and
 * LM head (the embedding matrix when tied_embeddings).                    */
typedef struct {
    int32_t n_layers;
    int32_t hidden;          /* H; n_q_heads * head_dim may differ (a tensor-parallel shard) */
    int32_t n_q_heads;
    int32_t n_kv_heads;      /* divides n_q_heads */
    int32_t head_dim;        /* D: 64 or 128 */
    int32_t ffn;             /* F */
    int32_t vocab;           /* V */
    float rms_eps;
    float rope_theta;
    int32_t tied_embeddings; /* 1: LM head reads the embedding matrix */
    int32_t batch;           /* B rows per step, 1..8, fixed per handle */
    int32_t max_seq;         /* KV slots per (layer, K/V, row, group) */
    int32_t device;          /* HIP device ordinal */
    int32_t n_cus;           /* 0 = every CU of the device; else a smaller grid */
    int32_t n_splits;        /* split-KV partitions per (row, KV group); 0 = auto */
    int32_t n_chunks;        /* K-chunks of the down projection; 0 = auto (2 for 2..4 batch rows
                                with ffn <= 8192, else 4) */
    uint32_t flags;          /* MK_FLAG_* */
} mk_config;

/* Threads per workgroup of the step kernels (one workgroup per CU): 8 compute
 * waves, 1 weight-loader wave, 1 gather wave.                             */
#define MK_STEP_THREADS 640

#define MK_FLAG_NONE 0u
#define MK_FLAG_PROFILE 1u  /* per-wave cycle counters, read with mk_get_profile */
#define MK_FLAG_TRACE 2u    /* per-instruction timeline, read with mk_get_trace */
#define MK_FLAG_FP8_WEIGHTS 4u /* every projection matrix and the LM head are packed as OCP FP8
                                  E4M3 codes with one fp32 scale per output row (fp32(max|w_row| /
                                  448), 1 for a zero row; code = E4M3 value nearest to
                                  fp32(w / scale), ties to even), half the bytes of bf16 plus 4
                                  bytes per row; the embedding lookup stays bf16.  Not
                                  combinable with MK_FLAG_PROFILE / MK_FLAG_TRACE. */
#define MK_FLAG_DEBUG_NAN 8u   /* debugging: before every step (mk_decode_step, _greedy,
                                  _multikernel, graph replays) the library overwrites the values
                                  of the step's activation scratch with NaN (the tagged words keep
                                  their previous step's tags, so waits are unchanged), the
                                  down-projection accumulators and the logits, and each
                                  workgroup fills its LDS with NaN at launch: a read of any of
                                  them before its write shows up as NaN logits.  One extra
                                  launch per step.                                         */

/* Per-layer weight pointers: arrays of n_layers DEVICE pointers held in HOST
 * memory.  Every tensor is bf16, row-major in the nn.Linear layout [out][in]:
 *   attn_norm[l], mlp_norm[l]: [H]
 *   wq[l]: [Hq*D][H]   wk[l], wv[l]: [Hkv*D][H]   wo[l]: [H][Hq*D]
 *   w_gate[l], w_up[l]: [F][H]   w_down[l]: [H][F]
 * embed: [V][H], final_norm: [H], lm_head: [V][H] (ignored when tied).      */
typedef struct {
    const void* embed;
    const void* final_norm;
    const void* lm_head;
    const void* const* attn_norm;
    const void* const* wq;
    const void* const* wk;
    const void* const* wv;
    const void* const* wo;
    const void* const* mlp_norm;
    const void* const* w_gate;
    const void* const* w_up;
    const void* const* w_down;
} mk_weights;

typedef struct mk_handle mk_handle;

/* Validates `cfg`, queries the device, builds the per-CU instruction queues
 * and the packed-weight layout, and allocates all library-owned device
 * memory (packed weights, queues, activation scratch, RoPE table).  On error
 * *out is set to NULL.  Shape limits: Hq*D <= 16384, Hq % Hkv == 0, D in {64,128},
 * (Hq/Hkv) divides 8, H and F multiples of 8, 1 <= batch <= 8.            */
int mk_create(const mk_config* cfg, mk_handle** out);

/* Copies the caller's weights (device pointers, see mk_weights) into the
 * library's packed layout on `stream`, then synchronises `stream`; the caller
 * may free its tensors afterwards.  May be called again to replace weights. */
int mk_load_weights(mk_handle* h, const mk_weights* w, void* stream);

/* Bytes of the caller-owned KV cache: bf16 [L][2 (K,V)][B][Hkv][max_seq][D],
 * K stored after RoPE.  Returns 0 for an invalid config.                  */
size_t mk_kv_cache_bytes(const mk_config* cfg);

/* One greedy-decode step for every batch row, as ONE kernel launch on
 * `stream` (asynchronous; no allocation, no host synchronisation).
 *   tokens    device int32[B], ids in [0, V)
 *   positions device int32[B], 0 <= p < max_seq; cache slots [0, p) of row b
 *             must hold that row's earlier K/V; the step writes slot p
 *   kv_cache  device buffer of mk_kv_cache_bytes(cfg)
 *   logits    device float32[B][V] (written)
 * Steps on one handle must be ordered on one stream: the handle's scratch is
 * reused by every step.  Out-of-range ids/positions are detected on device
 * before any work: the error is recorded (mk_get_device_error) and the step
 * writes neither logits nor KV cache.                                      */
int mk_decode_step(mk_handle* h, const int32_t* tokens, const int32_t* positions,
                   void* kv_cache, float* logits, void* stream);

/* mk_decode_step followed by greedy selection, in the same ONE launch:
 * the next token of each row is argmax_v logits[b][v] (the lowest index among
 * equal maxima; NaN never wins; a row without a number gives 0), written to
 * tokens[b], and positions[b] advances by one -- the loop of greedy
 * decoding (pages "Megakernels for Gemma 4" and "Why it only works at low
 * concurrency": the per-token interval of an agent loop).  Each CU reduces
 * its LM-head rows; the last CU to finish merges the per-CU results.  The
 * logits are written as by mk_decode_step.  Not for handles created with
 * MK_FLAG_PROFILE or MK_FLAG_TRACE (MK_ERR_STATE).  After a device error,
 * mk_get_device_error also resets the merge counter.                      */
int mk_decode_step_greedy(mk_handle* h, int32_t* tokens, int32_t* positions,
                          void* kv_cache, float* logits, void* stream);

/* Same arguments, results and ordering rules; the same op bodies launched
 * once per op and layer (6 * n_layers + 1 launches), ordered only by the
 * kernel boundaries.  For A/B comparison with mk_decode_step.             */
int mk_decode_step_multikernel(mk_handle* h, const int32_t* tokens, const int32_t* positions,
                               void* kv_cache, float* logits, void* stream);

/* Greedy selection after a step (outside the step kernel): one launch on
 * `stream` that sets tokens[b] = argmax_v logits[b][v] (the lowest index among
 * equal maxima) and positions[b] += 1 for every batch row, so that back-to-back
 * steps need no host work.  logits: device float32[B][V]; tokens, positions:
 * device int32[B] (the next step's inputs).  Asynchronous; NaN logits never
 * win a comparison (an all-NaN row yields token 0).  Greedy decoding is the
 * setting of the speed-of-light figures on the Gemma TPU megakernel page
 * (withhopper.com); the tie-break is torch.argmax's.  Uses a small per-handle
 * device scratch area (per-slice partial maxima and a per-row counter that
 * each call leaves at zero): calls on one handle must not overlap in time
 * (issue them on one stream).                                              */
int mk_greedy_advance(mk_handle* h, const float* logits, int32_t* tokens, int32_t* positions, void* stream);

/* Measurement support: reads `bytes` (a multiple of 16) at the 16-byte aligned
 * device address `buf` once, as 4 * n_cus workgroups of 512 threads with
 * 16-byte loads, eight in flight per thread, on `stream` (asynchronous; time
 * it with events).  `sink`: device memory of at least 4 bytes that the kernel
 * may write.  The floor of a decode step is the time to read every weight
 * once at the memory's read rate (the page "Megakernels: Deleting the Kernel
 * Boundary to Win Back Microseconds", section "Where the microseconds go");
 * this gives the rate the device actually sustains, next to its data-sheet
 * peak.  Needs no handle; MK_ERR_INVALID_ARG on null/unaligned arguments or
 * n_cus outside 1..4096.                                                   */
int mk_read_probe(const void* buf, size_t bytes, void* sink, int n_cus, void* stream);

/* Measurement support: enqueues n_launches (1..100000) launches of an empty
 * kernel with n_blocks (1..65536) workgroups of n_threads (1..1024) threads
 * on `stream`, so that their cost can be timed next to the per-op path's
 * launches (the per-launch overhead of the page "Megakernels: Deleting the
 * Kernel Boundary to Win Back Microseconds", section "Where the microseconds
 * go").  Needs no handle; MK_ERR_INVALID_ARG when out of range.            */
int mk_empty_launches(int n_launches, int n_blocks, int n_threads, void* stream);

/* A decode loop captured once as a HIP graph and replayed with one call.
 * mk_graph_create records n_steps (1..4096) greedy steps, each one decode
 * step followed by mk_greedy_advance's kernel, on a private stream of its
 * own and instantiates the graph; nothing runs until mk_graph_launch.  The
 * four device pointers are baked into the graph (same meaning as for
 * mk_decode_step; tokens and positions are advanced on device by every
 * step), so every replay continues from whatever they hold when it starts.
 * flags: 0 = the single-launch step; MK_GRAPH_MULTIKERNEL = the per-op
 * launches of mk_decode_step_multikernel (launch cost without the host's
 * launch path, the replay point next to "one launch, one interpreter" of the
 * megakernel page); MK_GRAPH_EMPTY = as many empty-kernel launches as the
 * per-op step has, with the step's grid shape, and no greedy kernel (the
 * graph launch overhead alone; the buffers are not touched);
 * MK_GRAPH_FUSED_GREEDY = each step one mk_decode_step_greedy launch (no
 * separate greedy kernel; not combinable with the other flags).  The graph
 * holds no memset nodes.  Replays on one handle must be ordered on one
 * stream, like steps.  *out is NULL on error.  MK_ERR_HIP when the runtime
 * refuses the capture (for instance of the cooperative single-launch step);
 * the handle stays usable.  The graph must be destroyed before its handle. */
#define MK_GRAPH_MULTIKERNEL 1u
#define MK_GRAPH_EMPTY 2u
#define MK_GRAPH_FUSED_GREEDY 4u /* each step is one mk_decode_step_greedy launch */
typedef struct mk_graph mk_graph;
int mk_graph_create(mk_handle* h, int32_t* tokens, int32_t* positions, void* kv_cache,
                    float* logits, int n_steps, uint32_t flags, mk_graph** out);
/* Enqueues one replay of the graph on `stream` (asynchronous). */
int mk_graph_launch(mk_graph* g, void* stream);
/* Frees the graph.  NULL is accepted. */
int mk_graph_destroy(mk_graph* g);

/* Batched prefill ("One Token, 2,400 Kernel Launches", opening section: the
 * prompt is one compute-bound pass, decode the token-by-token phase): runs
 * the model over positions 0 .. n_tokens-1 of every batch row.
 *   w:        the caller's bf16 weights, as for mk_load_weights (device
 *             pointers, 16-byte aligned); read during the call only.
 *   tokens:   device int32 [B][n_tokens], ids in [0, vocab).
 *   kv_cache: the caller's cache; slots [0, n_tokens) of every (layer, K/V,
 *             row, group) are written, bf16 rounded to nearest even.
 *   logits:   device fp32 [B][vocab], the last position's logits.
 * Equals mk_decode_step at positions 0 .. n_tokens-1 with the same tokens,
 * up to fp32 rounding order (the projections run on the fp32 matrix cores).
 * Positions go through the layers in chunks (attention reads the earlier
 * chunks' keys and values from the cache), as many per chunk as a workspace
 * of at most 512 MiB holds; the handle keeps that workspace between calls
 * and allocates only when a call needs a larger one.  Synchronous: waits for
 * `stream`.  MK_ERR_INVALID_ARG: null or unaligned pointer, n_tokens outside
 * [1, max_seq], or (after the run) a token outside [0, vocab) — its rows are
 * then computed from a zero embedding.  MK_ERR_UNSUPPORTED_SHAPE for an
 * MK_FLAG_FP8_WEIGHTS handle; MK_ERR_OOM when the workspace does not fit.  */
int mk_prefill(mk_handle* h, const mk_weights* w, const int32_t* tokens, int32_t n_tokens, void* kv_cache,
               float* logits, void* stream);

/* mk_prefill for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops): same arguments and results, but it
 * allocates nothing, does not synchronise, and runs in a static 64 MiB
 * scratch array that each device the library runs on holds until the process
 * ends (prompts longer than fit in one pass go through in chunks).  Every
 * call on one device shares that array: calls that overlap on one device
 * (other streams, other handles) race.  A token outside [0, vocab) is not
 * returned as a status: it is recorded in the handle's device error record
 * (code 2, read with mk_get_device_error) and its rows use a zero embedding.
 * MK_ERR_UNSUPPORTED_SHAPE when one position of every batch row needs more
 * than 64 MiB of fp32 rows (B * (2H + 2*Hq*D + 2*Hkv*D + 2F) * 4 bytes), and
 * for FP8 handles; MK_ERR_INVALID_ARG as mk_prefill.                       */
int mk_prefill_static(mk_handle* h, const mk_weights* w, const int32_t* tokens, int32_t n_tokens, void* kv_cache,
                      float* logits, void* stream);

/* Frees everything the handle owns.  NULL is accepted. */
int mk_destroy(mk_handle* h);

/* Static description of a status code. */
const char* mk_status_string(int status);

/* Text of the last error on this handle ("" if none); valid until the next
 * call on the handle.  With h == NULL: the last mk_create failure.        */
const char* mk_last_error(const mk_handle* h);

/* Device-side error record, written by the first workgroup that detects a
 * range violation or whose bounded wait expires.                          */
typedef struct {
    uint32_t code;       /* 0 none, 1 wait timeout, 2 token out of range, 3 position out of range */
    uint32_t workgroup;
    uint32_t pc;         /* instruction index in that workgroup's queue */
    uint32_t opcode;
    uint32_t wave;
    uint32_t detail;     /* op-specific (e.g. the awaited tag or the bad value) */
} mk_device_error;

/* Synchronises the handle's device, copies the error record to *out and
 * clears it.  Returns MK_OK, or MK_ERR_DEVICE when a record was present.  */
int mk_get_device_error(mk_handle* h, mk_device_error* out);

/* Ablation (measurement only): from the next mk_decode_step on, the
 * single-launch step runs a kernel build in which the arithmetic of one
 * opcode is switched off -- its weight units still stream through the rings
 * and unread, its inputs are still awaited and its tagged outputs still
 * written (zeros; the O and down projections pass the residual through), so
 * every dependency stays in place and the step time shows what that
 * component costs (page "Megakernels for Gemma 4": how much the step
 * shrinks when a component is switched off).  opcode: 0 = none (the normal
 * build again), 1 RMS+QKV+RoPE, 2 attention, 3 attention reduce, 4 O
 * projection, 5 RMS+up/gate, 6 down projection, 7 RMS+LM head.  The logits
 * are then not the model's.  bf16 handles without profiling or tracing only
 * (MK_ERR_STATE); mk_decode_step_greedy refuses to run while one is set.
 * Synchronises the device.                                                 */
int mk_set_ablation(mk_handle* h, int32_t opcode);

/* Watchdog of the bounded waits ("Megakernels: Deleting the Kernel Boundary
 * to Win Back Microseconds", section "The catch": a hand-rolled dependency
 * graph that is wrong hangs instead of failing).  Every wait in the step
 * kernels polls at most `spins` times (0 restores the default of 2^25, a few
 * seconds), then writes an error record with code 1 (the workgroup, queue
 * position, opcode, wave and what it waited for), raises an abort flag that
 * every other waiting wave sees, and the grid drains normally.  Synchronises
 * the device.  The setting stays with the handle.                          */
int mk_set_spin_limit(mk_handle* h, uint32_t spins);

/* Diagnostics: launches stage `stage` (0 .. 6L: six per layer in op order,
 * then the LM head) of the per-op path on its own, as one kernel on `stream`.
 * A stage whose producers did not run in the same step waits for inputs that
 * never arrive; with a small spin limit (mk_set_spin_limit) this exercises the
 * watchdog.  The handle's step counter advances, so nothing the launch writes
 * is taken for a later step's data; the KV slot of a QKV stage and the logits
 * of the LM-head stage may be overwritten.                                */
int mk_debug_stage(mk_handle* h, int32_t stage, const int32_t* tokens, const int32_t* positions,
                   void* kv_cache, float* logits, void* stream);

/* Per-wave cycle counters of the last step (handle created with
 * MK_FLAG_PROFILE): counters[(cu * 10 + wave) * 8 + k], 8 x uint64 per wave,
 * waves 0..7 compute, 8 the weight loader, 9 the gather wave (only k = 0).
 * Compute k: 0 cycles in the kernel,
 * 1 waiting for weight units, 2 waiting for tagged inputs, 3 in workgroup
 * barriers, 4 units read, 5 barriers passed, 6 barrier polls, 7 barriers
 * this wave completed last.  Loader k: 0 cycles in the kernel, 1 waiting for
 * DMA completion, 2 waiting for ring space, 3 units loaded, 4 unit-rows.
 * `n` is the capacity of `counters` in elements; synchronises the device.
 * Returns MK_ERR_STATE when profiling is off.                             */
int mk_get_profile(mk_handle* h, uint64_t* counters, size_t n);

/* Per-instruction timeline of the last step (handle created with
 * MK_FLAG_TRACE): records[i * 52 + k] for each instruction i of the
 * concatenated per-CU queues (mk_schedule_info.total_insts records), times
 * in ticks of the GPU's 100 MHz real-time clock, which all CUs share:
 *   k = 0: opcode | layer << 8 | a << 16 | b << 32 | cu << 48
 *          (a, b: batch row and KV group for attention, batch row and head
 *          for the reduce, chunk for the down projection)
 *   k = 1 + 6w .. 6 + 6w for compute wave w (0..7): start, inputs loaded,
 *          inputs ready, main loop done (before the epilogue or merge), end,
 *          ticks spent waiting for weight units.
 *   k = 49 .. 51: the gather wave's start on the instruction's inputs, all
 *          polled inputs current, inputs staged in LDS.
 * `n` is the capacity in elements; synchronises the device.  Returns
 * MK_ERR_STATE when tracing is off.                                        */
int mk_get_trace(mk_handle* h, uint64_t* records, size_t n);

/* Litmus test of the tagged-word dependency protocol across CUs, and a probe
 * of its cross-CU latency (the hazard that "Megakernels: Deleting the Kernel
 * Boundary to Win Back Microseconds", section "Correctness without the free
 * barrier", warns about: a consumer must never see data older than the
 * producer's store).  n_pairs (1..512) pairs of single-wave workgroups, pair
 * p = workgroups p and n_pairs + p (on the same XCD of the round-robin
 * dispatch exactly when n_pairs is a multiple of the XCD count), play
 * `rounds` (1..2^20) round trips of `words` (1..1024) tagged words each way,
 * written and polled with the step kernel's own store and load primitives;
 * every value that arrives with the round's tag is checked.  Polls give up
 * after spin_limit sleeps (a timeout ends that pair's run).  Writes, to the
 * HOST array result[3 + 3 * n_pairs]: [0] mismatched values, [1] timeouts,
 * [2] completed round trips, then per pair: ticks (100 MHz) the ping side
 * spent, ping XCC id, pong XCC id.  Allocates and frees its own buffers,
 * runs on a private stream and waits for it.                              */
int mk_litmus(int device, int32_t n_pairs, int32_t rounds, int32_t words, uint32_t spin_limit, uint32_t* result);

/* Host-only inspection of the schedule for `cfg` on `n_cus` CUs: builds it,
 * checks that every output row / unit is produced exactly once and that the
 * per-CU queues can complete (simulated in stage order).  Needs no GPU.   */
typedef struct {
    int32_t n_cus;
    int32_t n_splits;
    int32_t n_chunks;
    int32_t max_insts_per_cu;
    int64_t total_insts;
    int64_t packed_weight_bytes;   /* weight bytes streamed per step (incl. row padding to 1 KiB units) */
    int64_t max_stream_bytes_per_wave;
    int64_t min_stream_bytes_per_wave;
    int32_t launches_multikernel;
    int32_t valid;                 /* 1 if all checks passed */
} mk_schedule_info;

int mk_schedule_inspect(const mk_config* cfg, int32_t n_cus, mk_schedule_info* out);

/* Host-only self-test of the schedule validator (the hand-built dependency
 * graph is what "Megakernels: Deleting the Kernel Boundary to Win Back
 * Microseconds", section "The catch", names as the hard part to debug):
 * builds the schedule for `cfg` on `n_cus` CUs, plants one defect, and runs
 * the validator on the result, in the first queue (lowest CU) that has a place
 * for it.  mutation: 0 none; 1 the queue's first instruction duplicated into
 * the next CU's queue (an output produced twice); 2 its first up/gate
 * instruction removed (an output never produced); 3 its last down-projection
 * instruction swapped with the later-stage instruction that follows it (a
 * queue that waits on its own later work), caught by the
 * stage-order check; 4 the same defect with the stage-order check switched
 * off, so that only the dependency simulation can catch it (as a deadlock).
 * Returns MK_OK if the validator accepts the schedule, MK_ERR_UNSUPPORTED_SHAPE
 * with its message in mk_last_error(NULL) if it rejects it, MK_ERR_INVALID_ARG
 * for a bad argument or a schedule without a place for the defect.  Needs no GPU. */
int mk_schedule_selftest(const mk_config* cfg, int32_t n_cus, int32_t mutation);

#ifdef __cplusplus
}
#endif
#endif /* MK_H */
