/*
 * pmk.h — C ABI of the persistent batch-1 decode megakernel library for MI355X (gfx950).
 *
 * The library runs single-stream (batch 1) greedy decode of a dense Llama-style decoder as
 * ONE persistent, CU-resident kernel per decode call: every CU executes a static queue of
 * tasks (GEMV tiles, attention splits, LM-head tiles) that the host lowers from the model
 * into a task DAG synchronised by step-tagged data and epoch flags (or monotonic counters),
 * after a static validator has proved the schedule deadlock- and race-free.
 *
 * Sources of the design (pages, by title and section):
 *  - "AutoMegaKernel: A Statically-Checked Agent Harness for Self-Retargeting Megakernel
 *    Synthesis" (explainer), Method: Layer 0 (one cooperative block per compute unit running
 *    a local wait -> dispatch -> signal queue on monotonic counters), Layer 1 (GEMV, attention
 *    and RMSNorm instructions), Layer 2 (Schedule IR task DAG and ScheduleConfig), and the
 *    Safety Gate (acyclicity, satisfiable thresholds 1 <= t <= #producers, per-queue order,
 *    joined multi-producer counters, happens-before on memory, output reachability, reject
 *    before any launch).  Problem statement: the batch-1 latency floor is weight bytes over
 *    HBM bandwidth; per-op launches and graph replay keep op boundaries.
 *  - "Kog AI MI300X monokernel tutorial": the monokernel keeps the whole decode loop,
 *    including LM-head sampling and the EOS check, in one resident kernel with no host
 *    re-entry; batch-1 projections are GEMV on vector ALUs with dot2, not matrix cores;
 *    work is partitioned at compile time over a fixed CU grid; sentinel polling replaced
 *    atomic arrival counters.
 *  - "Netra Kernel" summary, details: a C-ABI runtime binds persistent and boundary buffers
 *    and launches on a caller-owned stream; kernels are chosen by an exact operation
 *    contract and anything outside it is rejected, not approximated; FP8 E4M3 block-scale
 *    weights and GQA attention over an FP8 KV cache.
 *
 * Conventions
 *  - Every call returns pmk_status (PMK_OK = 0).  No C++ exception crosses the ABI.
 *    pmk_last_error(ctx) gives a human-readable reason for the last failure on ctx.
 *  - Device work is asynchronous on the caller's stream (a hipStream_t passed as void*;
 *    NULL is the default stream).  Device-side failures (watchdog time-outs, NaN logits)
 *    surface through pmk_poll_error() after the caller has synchronised the stream.
 *  - The CALLER allocates all device memory (for example as torch uint8 tensors) with the
 *    sizes pmk_buffer_sizes() reports, and keeps it alive until pmk_destroy().  The library
 *    allocates only small host-side tables and a few-KB device copy of the schedule.
 *  - One thread at a time per context.  Contexts are independent.
 */
#ifndef PMK_H_
#define PMK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PMK_ABI_VERSION 6

typedef enum {
  PMK_OK = 0,
  PMK_ERR_INVALID_ARG = 1,      /* NULL pointer, bad size, misaligned buffer, bad enum */
  PMK_ERR_UNSUPPORTED = 2,      /* model outside the contract (biases, head_dim, GQA ratio, dtype) */
  PMK_ERR_SCHEDULE_INVALID = 3, /* the static validator rejected the schedule; see pmk_last_error */
  PMK_ERR_CAPACITY = 4,         /* position + steps would exceed max_seq */
  PMK_ERR_NOT_BOUND = 5,        /* buffers not bound, or weights / KV not loaded yet */
  PMK_ERR_HIP = 6,              /* a HIP runtime call failed; see pmk_last_error */
  PMK_ERR_TIMEOUT = 7,          /* a device wait exceeded its spin limit (pmk_poll_error) */
  PMK_ERR_NAN = 8,              /* NaN logits reached the greedy choice (pmk_poll_error) */
  PMK_ERR_DEVICE = 9            /* the device cannot co-schedule the grid, or is not gfx950 */
} pmk_status;

/* Storage formats.  INT8 and INT4 are weight-only formats (W8A16 / W4A16; passage: the
 * AutoMegaKernel explainer, results, which name weight-only int8 and int4 megakernels): symmetric
 * two's-complement codes with one bf16 scale per row and 128-column group, w = q * s, and the
 * activation operand of each linear layer taken in binary16. */
typedef enum {
  PMK_DT_F16 = 0,
  PMK_DT_BF16 = 1,
  PMK_DT_FP8_E4M3 = 2,
  PMK_DT_INT8 = 3, /* one signed byte per weight */
  PMK_DT_INT4 = 4  /* two per byte, the even column in the low nibble */
} pmk_dtype;

typedef enum {
  PMK_MODE_MEGAKERNEL = 0, /* one persistent cooperative launch per decode call */
  PMK_MODE_GRAPH = 1,      /* one captured hipGraph of per-op kernels, replayed once per step */
  PMK_MODE_PER_OP = 2      /* the same per-op kernels launched directly (no graph) */
} pmk_mode;

typedef enum {
  PMK_SYNC_FLAGS = 0,   /* whole-vector joins (the residual stream, q and the step's K/V row, the
                           attention output) carry a step tag in every value and the consumers
                           poll the data; the other joins (attention splits, gate/up, LM head)
                           give each producer an epoch flag word that waiters poll */
  PMK_SYNC_COUNTERS = 1 /* every join: producers add 1 to a shared monotonic counter; waiters poll
                           it (the tagged data is then read once) */
} pmk_sync_mode;

/* The operation contract.  Supported: no biases, untied embeddings, head_dim in {64, 128},
 * n_q_heads % n_kv_heads == 0, hidden, ffn, n_q_heads*head_dim multiples of 8 (16 for FP8 and
 * INT8, 32 for INT4), and (weight_dtype, kv_dtype) one of (F16, F16), (BF16, BF16),
 * (FP8_E4M3, FP8_E4M3), (INT8, BF16), (INT4, BF16).  FP8 weights use 128x128 fp32 block scales;
 * INT8 / INT4 weights one bf16 scale per row and 128-column group (the last group of a row may be
 * shorter), and their GEMVs round the activation vector to binary16 and accumulate in fp32.  The
 * embedding and norm gains of FP8, INT8 and INT4 models are BF16. */
typedef struct {
  int32_t n_layers;
  int32_t hidden;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t ffn;
  int32_t vocab;
  int32_t max_seq;        /* KV capacity in positions */
  float rms_eps;
  float rope_theta;
  int32_t weight_dtype;   /* pmk_dtype */
  int32_t kv_dtype;       /* pmk_dtype */
  int32_t has_bias;       /* must be 0 */
  int32_t tie_embeddings; /* must be 0 */
} pmk_model_config;

/* Structural knobs of the schedule (the ScheduleConfig of the pages).  Zero means default. */
typedef struct {
  int32_t n_cus;        /* grid size = number of queues (default: all CUs of the device) */
  int32_t sync_mode;    /* pmk_sync_mode (default FLAGS) */
  int32_t attn_splits;  /* split-KV chunks per KV head (default: n_cus / n_kv_heads, capped by max_seq/16) */
  int32_t prefetch;     /* 0 (default): a GEMV task issues the first 10 of its 16-byte weight loads
                           per lane before its dependency wait, and an O-projection task whose tile
                           fits in LDS copies all of it there (LDS-DMA) before its wait instead;
                           1: the register loads only; -1: every weight load after the wait */
  int32_t trace_steps;  /* steps kept in the per-task trace ring (default 0 = no trace buffer) */
  int64_t spin_limit;   /* polls before a wait gives up and aborts the launch (default 1<<22) */
  int32_t combine_parts;    /* COMBINE tasks per kv head, each over a range of its q heads (a divisor of
                               n_q_heads / n_kv_heads; default: the fewest that keep one combine's partials
                               under ~33 KiB while the O-projection tiles still fit in LDS) */
  int32_t combine_o_share;  /* O-projection rows on the queues that run a COMBINE: 0 automatic, 1 none,
                               2 half a share, 3 a full share */
  int32_t prefill_chunk;    /* prompt positions per chunk of the batched prefill: 0 = 512 (or max_seq
                               rounded up to 128 if smaller), a multiple of 128 up to 1024, or -1 = no
                               batched prefill (every prompt position runs as a teacher-forced decode
                               step) */
  int32_t prefill_ksplit;   /* K-halves of the batched prefill's O and down projections: 0 automatic (two
                               where their tiles would fill at most half the grid), 1 never, 2 always
                               (where K has at least eight 32-column steps) */
  int32_t combine_o_copy;   /* a COMBINE copies the O-projection tile of its queue's next task to LDS
                               before its own wait: 0 automatic (when an attention split holds at least
                               128 positions, where the copy hides behind the longer wait), 1 never,
                               2 always */
  int32_t reserved[3];      /* must be 0 */
} pmk_schedule_config;

typedef struct {
  uint64_t arena_bytes;     /* packed weights, gains, scales, RoPE table */
  uint64_t kv_bytes;        /* K and V caches: 2 * L * n_kv * seqcap * head_dim * elem, where
                               seqcap = max_seq rounded up to 32 (each half 256-byte aligned) */
  uint64_t workspace_bytes; /* activations, partials, flags, counters, trace */
} pmk_sizes;

/* Device pointers to the canonical tensors (row-major [out][in] for every linear weight):
 *   embed[V][H], final_norm[H], lm_head[V][H] (+ lm_head_scale: [ceil(V/128)][ceil(H/128)] fp32
 *   for FP8, [V][ceil(H/128)] bf16 for INT8 / INT4),
 *   layers: n_layers * 9 pointers, per layer in order
 *     wq[nq*hd][H], wk[nkv*hd][H], wv[nkv*hd][H], wo[H][nq*hd], w_gate[F][H], w_up[F][H],
 *     w_down[H][F], attn_norm[H], ffn_norm[H]
 *   layer_scales (FP8, INT8 and INT4 weights, else NULL): n_layers * 7 pointers, the scales of
 *     the 7 linear tensors, each [ceil(out/128)][ceil(in/128)] fp32 (FP8) or [out][ceil(in/128)]
 *     bf16 bits (INT8 / INT4).
 * 16-bit tensors are raw F16/BF16 bits; FP8 tensors are E4M3FN bytes; INT8 tensors are int8
 * [out][in]; INT4 tensors are bytes [out][in/2] (column 2j in the low nibble of byte j, 2j+1 in
 * the high one).  The host arrays of pointers are read during the call only. */
typedef struct {
  const void* embed;
  const void* final_norm;
  const void* lm_head;
  const void* lm_head_scale;
  const void* const* layers;
  const void* const* layer_scales;
} pmk_weight_ptrs;

/* Watchdog / device error record (pmk_poll_error). */
typedef struct {
  int32_t code;     /* pmk_status of the device failure, PMK_OK if none */
  int32_t cu;       /* queue that failed */
  int32_t task;     /* task index */
  int32_t counter;  /* counter it waited on */
  uint32_t expected;
  uint32_t seen;
} pmk_device_error;

typedef struct {
  int32_t n_tasks;
  int32_t n_counters;
  int32_t n_cus;
  int32_t attn_splits;
  int32_t max_tasks_per_cu;
  int32_t sync_mode;
  uint64_t hash;        /* FNV-1a of the serialized schedule (deterministic across runs) */
} pmk_schedule_info;

typedef struct pmk_ctx pmk_ctx;

/* Citations below name a page by its title and the section of it that defines the operation:
 *   [AMK] "AutoMegaKernel: A Statically-Checked Agent Harness for Self-Retargeting Megakernel
 *         Synthesis" (explainer page); [Kog] "Kog AI MI300X monokernel tutorial" (news page);
 *   [Netra] "Netra Kernel" summary page. */

/* Version of this ABI (PMK_ABI_VERSION), for a caller's compatibility check.
 * Passage: [Netra] details, "C ABI" runtime with fixed symbols.  No error case. */
int pmk_abi_version(void);
/* Static text for a status code (never NULL; unknown codes give "unknown status"). */
const char* pmk_status_str(pmk_status s);
/* Text of the last failure on ctx (never NULL; empty when none).  Valid until the next call. */
const char* pmk_last_error(const pmk_ctx* ctx);
/* Text of the last failure of a call that could not return a context (pmk_create). */
const char* pmk_last_global_error(void);

/* Create a context.  Host only.
 * Passages: [Netra] details (kernels are selected by the operation's exact contract: shapes, data
 * formats, accumulation order, layout; a request outside it is rejected, never approximated);
 * [AMK] Method, Layer 2 (the model is lowered into a typed task DAG shaped by a ScheduleConfig) and
 * Safety Gate (the schedule is checked statically before any launch and rejected if it fails).
 * cfg: the model (read during the call only); sched: NULL for the defaults; hip_device: the HIP
 * device index, or < 0 for a device-less context (schedule inspection only; every device call on it
 * returns PMK_ERR_NOT_BOUND).  On success *out owns a new context (release with pmk_destroy).
 * Errors: PMK_ERR_INVALID_ARG (NULL cfg/out), PMK_ERR_UNSUPPORTED (outside the contract),
 * PMK_ERR_SCHEDULE_INVALID (the validator rejected the lowering), PMK_ERR_DEVICE (not gfx950, no
 * cooperative launch, or the kernel cannot be resident), PMK_ERR_HIP; the reason is in
 * pmk_last_global_error().  Nothing is allocated on the device. */
pmk_status pmk_create(const pmk_model_config* cfg, const pmk_schedule_config* sched, int hip_device,
                      pmk_ctx** out);
/* Release a context (NULL is ignored).  The caller's buffers are not freed.  Passage: [Netra]
 * details (the runtime binds caller buffers; ownership stays with the caller). */
void pmk_destroy(pmk_ctx* ctx);

/* Bytes of the three caller-allocated device buffers (arena, KV cache, workspace).
 * Passage: [Netra] details (the engine carries a static memory and layout plan; the runtime only
 * binds buffers).  Errors: PMK_ERR_INVALID_ARG for NULL arguments. */
pmk_status pmk_buffer_sizes(const pmk_ctx* ctx, pmk_sizes* out);
/* Bind caller-owned device buffers.  Non-owning: they must stay allocated until pmk_destroy or the
 * next bind.  arena, kv and workspace must be 256-byte aligned device pointers of at least the
 * reported sizes.  Uploads the schedule tables and clears the synchronisation state (synchronous).
 * Passage: [Netra] details (the runtime links persistent and boundary buffers, then launches on a
 * caller-owned stream).  Errors: PMK_ERR_INVALID_ARG (NULL or misaligned), PMK_ERR_NOT_BOUND
 * (device-less context), PMK_ERR_HIP.  Weights and KV state must be loaded again after a bind. */
pmk_status pmk_bind(pmk_ctx* ctx, void* d_arena, void* d_kv, void* d_workspace);

/* pmk_bind for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the workspace is the library's own static device
 * array of at most 32 MiB per device (held by each device that loads the library until the process
 * ends), so only the arena and the KV cache are the caller's.  The call allocates nothing (no
 * hipMalloc, hipFree or allocating library routine); like pmk_bind it uploads the schedule tables
 * and clears the synchronisation state, so nothing of an earlier user of the array carries over.
 * One context per device at a time: a later pmk_bind_static_workspace on the same device takes the
 * array over, and device calls on the context that held it before then fail with
 * PMK_ERR_NOT_BOUND; calls of two contexts on one device's array that overlap in time race.
 * Errors: PMK_ERR_CAPACITY (the schedule's workspace exceeds the array: larger models, a trace
 * ring or the batched prefill's chunk buffers of a large model need pmk_bind, or a context created
 * with prefill_chunk = -1), PMK_ERR_INVALID_ARG, PMK_ERR_NOT_BOUND (device-less context),
 * PMK_ERR_DEVICE, PMK_ERR_HIP. */
pmk_status pmk_bind_static_workspace(pmk_ctx* ctx, void* d_arena, void* d_kv);

/* Repack the canonical tensors into the arena (QKV rows concatenated with each RoPE pair made
 * adjacent, gate/up rows interleaved, gains widened to fp32, RoPE cos/sin table; INT8 / INT4 codes
 * re-encoded for the kernels' conversion to binary16: offset binary, int4 nibbles reordered within
 * each 32-bit word).
 * Passages: [Netra] details (weight layout and FP8 E4M3 block-scale semantics are fixed ahead of
 * time); [AMK] Method (HF Llama-family models are imported into the schedule).
 * src: device pointers to the canonical tensors (pmk_weight_ptrs; the host arrays are read during
 * the call only).  Asynchronous on `stream` (a hipStream_t, NULL = default stream); the sources may
 * be freed once the stream has synchronised.  Errors: PMK_ERR_NOT_BOUND, PMK_ERR_INVALID_ARG
 * (missing pointers or scales), PMK_ERR_HIP. */
pmk_status pmk_load_weights(pmk_ctx* ctx, const pmk_weight_ptrs* src, void* stream);

/* Teacher-forced prefill: runs positions 0..P-1 from d_tokens[P] (device int32), writing the KV
 * cache; the greedy choice after the last position becomes the next input token (and is also
 * stored to d_first_token, a device int32, if not NULL).
 * Passages: [Kog] how the monokernel removes kernel-launch overhead (prefill, decode, LM-head
 * sampling and the EOS check run in the resident program); [Netra] details (GQA attention over an
 * FP8 KV cache, with its scale semantics fixed by the contract).
 * FP8 KV cache: d_kv_scales [n_layers][n_kv][2] (K, V) fp32 device array gives static scales; with
 * NULL the library derives them from this prompt: a calibration pass with every scale 1 records the
 * largest |k| and |v| per (layer, kv head), each scale becomes that maximum / 448 in fp32 (1 if the
 * maximum is 0), and the prefill then runs with those scales (read them back with pmk_get_kv_scales).
 * Other KV formats ignore d_kv_scales.  Unless prefill_chunk is -1, positions 0..P-2 run batched,
 * in chunks of prefill_chunk tokens, in ONE cooperative launch of grid-wide phases (RMSNorm, QKV
 * GEMM + RoPE + KV append, causal attention, O GEMM, RMSNorm, gate/up GEMM + SwiGLU, down GEMM)
 * with the GEMMs on the matrix cores (activations as two 16-bit terms, within 2^-18 of fp32;
 * binary16 ones for INT8 / INT4, as the format defines; the O and down projections in two
 * K-halves as prefill_ksplit says), and the last position as a teacher-forced decode step; with -1 every
 * position runs as a teacher-forced decode step.  Resets the position and the synchronisation
 * state.
 * Asynchronous on `stream`.  Errors: PMK_ERR_NOT_BOUND (no weights), PMK_ERR_INVALID_ARG (NULL
 * tokens, P <= 0), PMK_ERR_CAPACITY (P > max_seq), PMK_ERR_HIP; a batched-prefill barrier that
 * exceeds spin_limit polls records PMK_ERR_TIMEOUT for pmk_poll_error. */
pmk_status pmk_prefill_kv(pmk_ctx* ctx, const int32_t* d_tokens, int32_t P, const float* d_kv_scales,
                          int32_t* d_first_token, void* stream);

/* Copy the FP8 KV scales in force, [n_layers][n_kv][2] (K, V) fp32, to the device array d_out.
 * Passage: [Netra] details (FP8 KV attention with explicit scale semantics).  Asynchronous on
 * `stream`.  Errors: PMK_ERR_INVALID_ARG (NULL d_out, or a KV cache that is not FP8),
 * PMK_ERR_NOT_BOUND, PMK_ERR_HIP. */
pmk_status pmk_get_kv_scales(pmk_ctx* ctx, float* d_out, void* stream);

/* Resume from saved state: copies KV contents d_k, d_v [n_layers][n_kv][P][head_dim] (cache
 * element format, device) into positions 0..P-1, sets the position to P and the next input token to
 * `next_token`.  d_kv_scales as for pmk_prefill_kv, but required for an FP8 cache (the contents are
 * already quantised).  Passage: [Netra] details (persistent buffers bound by the runtime; FP8-KV
 * scale semantics).  Asynchronous.  Errors: PMK_ERR_CAPACITY (P > max_seq), PMK_ERR_INVALID_ARG
 * (missing pointers or scales, next_token outside the vocabulary), PMK_ERR_NOT_BOUND, PMK_ERR_HIP. */
pmk_status pmk_load_kv(pmk_ctx* ctx, const void* d_k, const void* d_v, int32_t P, int32_t next_token,
                       const float* d_kv_scales, void* stream);

/* Save state: copies positions 0..P-1 of the KV cache (P <= the current position) to d_k, d_v
 * [n_layers][n_kv][P][head_dim] in the cache element format (device), the layout pmk_load_kv takes.
 * Passage: [Netra] details (persistent buffers the runtime binds; here the cache contents leave the
 * library in the canonical layout).  Asynchronous on `stream`.  Errors: PMK_ERR_NOT_BOUND (no KV
 * state), PMK_ERR_INVALID_ARG (P outside [0, position], missing pointers), PMK_ERR_HIP. */
pmk_status pmk_read_kv(pmk_ctx* ctx, void* d_k, void* d_v, int32_t P, void* stream);

/* Rewind to position `pos` (0 < pos <= current position) with the next input token read from
 * d_token (device int32).  KV entries at positions >= pos are overwritten by later steps.  After a
 * decode call with an eos id this first reads the exact position from the device (synchronising).
 * Passage: [AMK] Results (teacher-forced and greedy runs from the same state are compared).
 * Errors: PMK_ERR_INVALID_ARG (pos outside (0, position], NULL token), PMK_ERR_NOT_BOUND. */
pmk_status pmk_rewind(pmk_ctx* ctx, int32_t pos, const int32_t* d_token, void* stream);

/* n greedy decode steps from the next-token slot at the current position.  Step i consumes the
 * current input token at position pos+i, appends its K and V, and writes the greedy next token to
 * d_out_tokens[i] (device int32 [n]); with d_out_logits != NULL the fp32 logits go to
 * d_out_logits[i*vocab ...] (device).  eos_id >= 0 stops after the step that emits it; the number of
 * steps run goes to *d_n_done (device int32, may be NULL).  MEGAKERNEL mode is ONE kernel launch;
 * GRAPH mode replays one captured graph of per-op kernels per step; PER_OP launches them directly.
 * Passages: [Kog] how the monokernel removes kernel-launch overhead (the whole decode loop, LM-head
 * sampling and the EOS check stay in one resident kernel with no host re-entry); [AMK] Problem
 * (batch-1 decode is bandwidth bound: the floor is weight bytes over HBM bandwidth) and Method,
 * Layer 0 (one cooperative block per compute unit runs its queue: wait, dispatch, signal).
 * Asynchronous on `stream`; the host does not re-enter during the call.  The position advances by
 * the steps run (after an eos stop the device keeps the exact position; pmk_get_position reads it).
 * Errors: PMK_ERR_NOT_BOUND (weights or KV state missing), PMK_ERR_INVALID_ARG (n <= 0, NULL
 * d_out_tokens), PMK_ERR_CAPACITY (position + n > max_seq), PMK_ERR_HIP.  Device-side failures
 * (watchdog time-out, NaN logits) are reported by pmk_poll_error. */
pmk_status pmk_decode_n_tokens(pmk_ctx* ctx, int32_t n, int32_t* d_out_tokens, float* d_out_logits,
                               int32_t eos_id, int32_t* d_n_done, void* stream);

/* Execution mode (pmk_mode) of later calls.  Passages: [AMK] Problem (per-op launches and graph
 * replay keep the operator boundaries the megakernel removes); [Netra] details (a HIP graph
 * prepared at initialisation is replayed).  Errors: PMK_ERR_INVALID_ARG for an unknown mode. */
pmk_status pmk_set_mode(pmk_ctx* ctx, int32_t mode);
/* Current position (next position to be written).  After a decode call with an eos id this
 * synchronises the device and reads the exact position.  Errors: PMK_ERR_INVALID_ARG (NULL). */
pmk_status pmk_get_position(const pmk_ctx* ctx, int32_t* pos);

/* After the caller synchronised the stream: reads the device error word into *err (may be NULL) and
 * returns its code (PMK_ERR_TIMEOUT: a wait exceeded its spin limit; PMK_ERR_NAN: NaN logits).
 * Passage: [AMK] Safety Gate (an unsafe schedule must not stall the GPU: every wait here is
 * bounded by a watchdog that aborts the launch instead). */
pmk_status pmk_poll_error(pmk_ctx* ctx, pmk_device_error* err);

/* Trace: with trace_steps > 0 and pmk_set_trace(ctx, 1) (which clears the ring), each task of
 * the first trace_steps steps of the next decode call records its wait begin, start and end, and
 * up to four task-specific sub-phase stamps (GEMV: input staged, rows done; attention: scores
 * done, partial stored; combine: partials loaded), from the constant 100 MHz clock.
 * pmk_trace_export writes Chrome-trace JSON (synchronises the device); pmk_trace_stats gives the
 * mean share of queue time spent waiting and the mean step time.
 * Passage: [Kog] how the monokernel removes kernel-launch overhead (synchronisation is measured as
 * a share of token time).  Errors: PMK_ERR_INVALID_ARG (no trace buffer, unwritable path). */
pmk_status pmk_set_trace(pmk_ctx* ctx, int32_t on);
pmk_status pmk_trace_export(pmk_ctx* ctx, const char* json_path);
pmk_status pmk_trace_stats(pmk_ctx* ctx, double* wait_share, double* step_us);

/* Result of pmk_tune. */
typedef struct {
  int32_t tried;          /* candidate schedules built */
  int32_t kept;           /* candidates kept (each faster than the best before it by more than 0.2%) */
  int32_t gate_rejected;  /* candidates whose outputs failed the correctness gate */
  int32_t invalid;        /* candidates the validator, the workspace capacity or LDS refused */
  double us_before;       /* µs per step of the measured steps on the schedule in force before */
  double us_after;        /* the same on the schedule chosen */
  pmk_schedule_config chosen;  /* the knobs in force after tuning (combine_parts, attn_splits resolved) */
  char desc[232];         /* the changes kept, e.g. "gate/up rows per XCD x1.0; combine_o_share 3" */
} pmk_tune_result;

/* Schedule tuning: a keep-or-revert search over the ScheduleConfig knobs and the GEMV row shares.
 * Passage: [AMK] Autoresearch loop (propose a ScheduleConfig change, validate it, check correctness
 * against a reference, time it, keep it or revert) and Results (tuned schedules over the default
 * configuration).  From the current position and next input token, the schedule in force is timed
 * on `steps` megakernel steps (default 32, at most 64; HIP events, after an untimed pass of the same
 * steps from the same state); then, one at a time, candidates are built, validated (Safety Gate),
 * installed and timed the same way: gate/up and down row shares weighted by the streaming rate each
 * queue measured in a traced run (grouped per queue or per XCD, the XCD id each workgroup read from
 * the hardware, moved fully or half-way from even), the O-projection rows on the combine queues
 * (none, half, full), the combines per kv head and fewer attention splits.  A candidate is kept if
 * it emits the same greedy token at every measured step as the starting schedule, with the same
 * largest logit within 1e-3 (a schedule change only regroups partial sums; 2e-2 for INT8 / INT4,
 * whose binary16 operand rounding moves some elements by a whole step when a sum regroups), and is
 * faster than the best so far by more than 0.2%; otherwise the best schedule is reinstalled.
 * Rate-based candidates
 * need a context created with trace_steps >= 2.  Every schedule change clears the synchronisation
 * state; the position and next token are restored (KV rows past the position are rewritten by the
 * next decode).  Synchronous on `stream`.  *result may be NULL.  Errors: PMK_ERR_NOT_BOUND,
 * PMK_ERR_CAPACITY (position + steps > max_seq), PMK_ERR_SCHEDULE_INVALID, PMK_ERR_HIP, or a
 * device error of a measured run. */
pmk_status pmk_tune(pmk_ctx* ctx, int32_t steps, pmk_tune_result* result, void* stream);

/* Schedule inspection (host only, also for device-less contexts).  Passage: [Netra] details
 * (deterministic engine artifacts: the schedule hash is reproducible across runs).
 * Errors: PMK_ERR_INVALID_ARG for NULL arguments. */
pmk_status pmk_schedule_get_info(const pmk_ctx* ctx, pmk_schedule_info* info);

/* ---- Schedule IR, exposed for the validator's tests and the validator CLI ----
 * Passage for this whole block: [AMK] Method, Layer 2 (the model lowered into a typed Schedule IR:
 * a task DAG over per-compute-unit queues synchronised by monotonic counters) and Safety Gate (the
 * static checks run on that IR before any launch).  Host only; no device is needed. */
typedef enum {
  PMK_OP_QKV = 1,     /* RMSNorm prologue + packed QKV GEMV rows [a0,a1) + RoPE + KV append */
  PMK_OP_ATTN = 2,    /* split-KV attention partial (max, sum, P.V) for kv head a0, split a1 */
  PMK_OP_OPROJ = 3,   /* O GEMV rows [a0,a1) + residual */
  PMK_OP_GATEUP = 4,  /* RMSNorm prologue + interleaved gate/up GEMV rows [a0,a1) + SwiGLU */
  PMK_OP_DOWN = 5,    /* down GEMV rows [a0,a1) + residual */
  PMK_OP_LMHEAD = 6,  /* final RMSNorm + LM-head rows [a0,a1) + tile argmax into the step key */
  PMK_OP_TOKEN = 7,   /* reads the step key, writes the output token and the next-input slot */
  PMK_OP_COMBINE = 8  /* merges the attention partials of every split of kv head a0 into o, for the
                         group's q heads [a1 & 255, a1 >> 8) */
} pmk_op;

typedef struct {
  int32_t op;          /* pmk_op */
  int32_t layer;
  int32_t a0, a1;
  int32_t wait_ctr;    /* counter index, or -1 */
  int32_t wait_count;  /* threshold within one step: 1 <= t <= producers(wait_ctr) */
  int32_t wait_lag;    /* 0: producers of the same step; 1: of the previous step.  At global step e
                          the wait needs counter >= (e - lag) * producers + wait_count (flags mode:
                          at least wait_count producer flags >= e - lag + 1). */
  int32_t signal_ctr;  /* counter index, or -1 */
  int32_t signal_slot; /* this producer's flag slot in signal_ctr */
} pmk_task;

typedef struct pmk_schedule pmk_schedule;

/* Build the schedule for `n_cus` queues without a device ([AMK] Method, Layer 2: lowering with a
 * ScheduleConfig).  *out owns a new schedule (pmk_schedule_free).  Errors: PMK_ERR_INVALID_ARG,
 * PMK_ERR_UNSUPPORTED (outside the contract), PMK_ERR_SCHEDULE_INVALID (the lowering failed). */
pmk_status pmk_schedule_build(const pmk_model_config* cfg, const pmk_schedule_config* sched, int32_t n_cus,
                              pmk_schedule** out);
/* The same with per-queue row weights for the GEMV phases: weights[op * n_cus + q] for pmk_op op
 * (QKV, OPROJ, GATEUP, DOWN, LMHEAD; other rows of the 8 x n_cus array are ignored), positive; each
 * GEMV task's rows are proportional to its queue's weight (at least one row or row pair each).
 * ([AMK] Method, Layer 2: CU allocation is a ScheduleConfig knob.)  Errors as pmk_schedule_build,
 * and PMK_ERR_INVALID_ARG for a weight that is not positive. */
pmk_status pmk_schedule_build_weighted(const pmk_model_config* cfg, const pmk_schedule_config* sched, int32_t n_cus,
                                       const float* weights, pmk_schedule** out);
/* Accessors and editors of the IR ([AMK] Method, Layer 2: the schedule is the edit surface that
 * proposals change; Safety Gate: every edited schedule is re-validated before use).  NULL or an
 * index out of range gives PMK_ERR_INVALID_ARG (or 0 / -1 / NULL for the value-returning ones). */
void pmk_schedule_free(pmk_schedule* s);
int32_t pmk_schedule_num_tasks(const pmk_schedule* s);
int32_t pmk_schedule_num_counters(const pmk_schedule* s);
int32_t pmk_schedule_num_queues(const pmk_schedule* s);
pmk_status pmk_schedule_get_task(const pmk_schedule* s, int32_t i, pmk_task* t);
pmk_status pmk_schedule_set_task(pmk_schedule* s, int32_t i, const pmk_task* t);
/* queue q's task list; *len receives its length; returns a pointer into the schedule */
const int32_t* pmk_schedule_queue(const pmk_schedule* s, int32_t q, int32_t* len);
pmk_status pmk_schedule_set_queue(pmk_schedule* s, int32_t q, const int32_t* tasks, int32_t len);
int32_t pmk_schedule_counter_producers(const pmk_schedule* s, int32_t c);
pmk_status pmk_schedule_set_counter_producers(pmk_schedule* s, int32_t c, int32_t producers);
/* Static validator ([AMK] Safety Gate: deadlock-freedom, race-freedom, correctness): returns PMK_OK
 * or PMK_ERR_SCHEDULE_INVALID with the first failed check (one line, "<check>: <detail>") copied
 * into report[0..cap). */
pmk_status pmk_schedule_validate(const pmk_schedule* s, char* report, size_t cap);
/* CPU simulator ([AMK] Safety Gate, checked dynamically): executes the queues for `steps` steps
 * with one host thread per queue and randomised yields, treating each task as reading/writing its
 * declared regions in poisoned stamp buffers.  Returns PMK_OK, PMK_ERR_TIMEOUT (a queue stuck:
 * deadlock), PMK_ERR_SCHEDULE_INVALID (a read observed a poisoned or stale value: race) or
 * PMK_ERR_INVALID_ARG (NULL, steps <= 0, or a model too large to simulate). */
pmk_status pmk_schedule_simulate(const pmk_schedule* s, int32_t steps, uint64_t seed, char* report, size_t cap);
/* FNV-1a hash of the serialised schedule ([Netra] details: deterministic artifacts); 0 for NULL. */
uint64_t pmk_schedule_hash(const pmk_schedule* s);

#ifdef __cplusplus
}
#endif
#endif /* PMK_H_ */
