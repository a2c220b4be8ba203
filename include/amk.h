/*
 * amk.h - C ABI of the persistent decode megakernel library (libamk.so) for AMD MI355X (gfx950).
 *
 * One call of amk_decode_step runs one autoregressive decode step of a Llama-style decoder
 * (RMSNorm, QKV projection, RoPE, grouped-query attention over a bf16 KV cache, O projection,
 * SwiGLU MLP, final norm, LM head, greedy argmax).
 *
 * Source of the operation: the Ada-MK technical summary (gist.science, "Methodology": a decode
 * step of the Transformer decoder plus LM head fused into one persistent kernel whose execution
 * order is searched offline and solidified, "Phase I"; warp-specialised execution, "Phase II")
 * and the AutoMegaKernel abstract (page 5 of the set: a HuggingFace Llama-family model compiled
 * into one persistent kernel, a frozen schedule IR checked statically for deadlock and races
 * before launch, int8 W8A16 weights, greedy decoding).
 *
 * Conventions for every entry point:
 *   - every function returns amk_status; no C++ exception crosses this boundary;
 *   - argument errors are reported synchronously, before anything is launched;
 *   - on failure amk_last_error() returns a message for the calling thread;
 *   - "device" pointers are HIP device memory of the current device; "host" pointers are
 *     ordinary process memory; `stream` is a hipStream_t passed as void* (NULL = default stream).
 * Threading: a model may be used from one thread (or serialised by the caller) at a time.
 */
#ifndef AMK_H
#define AMK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  AMK_OK = 0,
  AMK_E_INVALID = 1,            /* bad argument or shape */
  AMK_E_UNSUPPORTED = 2,        /* valid request this build does not implement */
  AMK_E_OOM = 3,                /* device or host allocation failed */
  AMK_E_SCHEDULE_REJECTED = 4,  /* the schedule failed static validation; nothing launched */
  AMK_E_HIP = 5,                /* a HIP runtime call failed (message carries its text) */
  AMK_E_CAPACITY = 6,           /* position or batch beyond what was allocated */
  AMK_E_DEVICE_TIMEOUT = 7,     /* a device-side dependency wait exceeded its bound */
  AMK_E_DEVICE_FAULT = 8        /* the device flagged bad data (e.g. token id out of range) */
} amk_status;

/* Weight formats (the Ada-MK technical summary, "Key Contributions" item 4, quantises to GPTQ
 * W4A16; W8A16 and bf16 are the other two). Activations are floating point in every format. */
typedef enum { AMK_WT_BF16 = 0, AMK_WT_INT8 = 1, AMK_WT_INT4 = 2 } amk_wtype;

typedef enum {
  AMK_PATH_MEGAKERNEL = 0,  /* one persistent launch per step, frozen per-CU task tables */
  AMK_PATH_UNFUSED = 1      /* ablation: one kernel launch per operator (1 + 10 L + 3 per step) */
} amk_path;

/* Model shape. hidden = n_heads * head_dim; n_heads % n_kv_heads == 0; head_dim even and a
 * multiple of 8; hidden and ffn multiples of 8; 1 <= max_batch <= 16. */
typedef struct {
  int32_t n_layers, hidden, n_heads, n_kv_heads, head_dim, ffn, vocab;
  float rms_eps, rope_theta;
  int32_t tied_lm_head; /* 1: the LM head is the embedding matrix */
  int32_t wtype;        /* amk_wtype of the 7 layer matrices and the (untied) LM head */
  int32_t max_batch;    /* largest batch a decode step will be called with */
  int32_t max_seq;      /* largest position + 1 the model will be asked to decode */
  int32_t group_size;   /* AMK_WT_INT4: inputs per scale group (a multiple of 32 dividing hidden
                         * and ffn); must be 0 for the other formats */
} amk_config;

/* Per-layer weights: device pointers, [out, in] row-major. bf16 matrices hold bfloat16 bit
 * patterns; int8 matrices hold int8 values with one float32 scale per output row (s* arrays,
 * NULL for bf16); int4 matrices are uint8 [out, in / 2], byte j of a row holding input 2j in its
 * low and 2j + 1 in its high nibble (4-bit two's complement, -8..7), with float32 scales
 * [out, in / group_size]: W[o][i] = s[o][i / group_size] * q[o][i]. Norm gains are bfloat16
 * [hidden]. */
typedef struct {
  const void *wq, *wk, *wv, *wo, *wg, *wu, *wd;
  const float *sq, *sk, *sv, *so, *sg, *su, *sd;
  const void *attn_norm, *mlp_norm;
} amk_layer_weights;

/* embed: bf16 [vocab, hidden]; final_norm: bf16 [hidden]; lm_head: [vocab, hidden] (bf16, int8
 * with lm_head_scale [vocab], or int4 packed as above with lm_head_scale
 * [vocab, hidden / group_size]) or NULL when tied (bf16 only). `layers` is a HOST array of n_layers
 * entries. */
typedef struct {
  const void *embed, *final_norm, *lm_head;
  const float *lm_head_scale;
  const amk_layer_weights *layers;
} amk_weights;

/* Schedule-search parameters (host only). Zero fields select the builder's default. */
typedef struct {
  int32_t attn_blocks;   /* KV blocks per KV head (split-KV); 0 = auto */
  int32_t min_block;     /* smallest KV block (positions) the auto choice may produce; 0 = 64 */
  int32_t placement;     /* 0 = XCD-blocked (tiles of one KV group on one XCD), 1 = round-robin */
  int32_t rotate;        /* phase-to-phase CU rotation of tile placement (0 = none) */
  int32_t ctx_hint;      /* context length the cost model assumes (0 = max_seq) */
  int32_t min_tile_kb;   /* smallest weight tile (KiB) a GEMV is cut into; 0 = 4 */
  int32_t search;        /* 1: exhaustive search over the free fields above; 0: take them as is */
  int32_t heads_per_task; /* query heads per attention task, a divisor of the heads sharing a KV
                           * head: 0 = auto (models of batch capacity 1: a group's heads split so
                           * that up to two attention tasks run per CU; otherwise whole groups) */
} amk_sched_params;

/* Cost model used by the schedule search (host only). Zero fields select defaults: the model
 * amk_calibrate measured, stored as JSON in cost_model.json beside libamk.so (or the file named by
 * the AMK_COST_MODEL environment variable; "off" skips it) when its CU count matches, else built-in
 * values. */
typedef struct {
  double cu_stream_gbs;  /* sustained HBM read rate of one CU when all CUs stream, GB/s */
  double hop_us;         /* latency from a producer's last store to a consumer's start, us */
  double task_us;        /* fixed cost of one task beyond its hop and its bytes, us */
  double l2_gbs;         /* per-CU rate for re-read activation data (L2 / MALL), GB/s */
  double prefetch_kb;    /* weight bytes a batch-1 GEMV tile streams before its wait, KiB */
  double attn_us;        /* fixed cost of an attention block's partial beyond its hop and bytes, us */
} amk_cost_model;

typedef struct {
  int32_t n_cu;              /* compute units the schedule targets (grid size) */
  int32_t n_tasks;           /* tasks per step */
  int32_t launches_per_step; /* kernel launches one amk_decode_step issues */
  int32_t lds_bytes;         /* LDS per workgroup of the megakernel */
  int32_t attn_blocks;       /* KV blocks per KV head */
  int32_t path;              /* amk_path */
  uint64_t weight_bytes;     /* algorithmic weight bytes read per step (matrices, gains, scales) */
  double predicted_us;       /* cost-model makespan of the frozen schedule at ctx_hint */
  uint64_t scratch_bytes;    /* device scratch of one decode step: flags, step counter, activation
                              * slots, attention partials, logits (one block, owned by the model) */
  int32_t heads_per_pass;    /* query heads one attention pass of the model's kernels processes:
                              * the megakernel instance fitted to the schedule's head ranges, or
                              * the operator kernels' whole-group passes */
} amk_model_info;

typedef struct amk_model amk_model;
typedef struct amk_kv amk_kv;

/* Create a model on the current device: the decoder compiled into one persistent kernel that runs
 * a frozen, statically checked schedule (AutoMegaKernel abstract; Ada-MK technical summary,
 * "Methodology", Phase I, the execution path solidified offline). Weights are BORROWED for the
 * duration of the call: the
 * library repacks them into its own buffers and synchronises `stream` before returning, so the
 * caller may free them afterwards. The packed rows keep RoPE pairs and gate/up pairs adjacent.
 * A model of max_batch 1 keeps those rows row-major. A larger max_batch stores each matrix
 * tile-major (16 rows x 32 inputs per contiguous tile, the matrix cores' step), which is why its
 * schedules cut GEMVs on 16-row boundaries. schedule_blob (host, may be NULL)
 * is a frozen schedule from amk_schedule_build; NULL builds one with default parameters. The
 * schedule is validated before anything is launched (AMK_E_SCHEDULE_REJECTED on failure). */
amk_status amk_model_create(const amk_config *cfg, const amk_weights *weights, int32_t path,
                            const void *schedule_blob, size_t blob_bytes, void *stream,
                            amk_model **out);

/* Bytes of a KV cache for `batch` sequences of `max_seq` positions (the cache the decode step
 * attends over; the pages fix no layout, this is the library's):
 * layout [n_layers][2 (K, V)][batch][n_kv_heads][max_seq][head_dim] bfloat16, K post-RoPE. */
amk_status amk_kv_bytes(const amk_model *m, int32_t batch, int32_t max_seq, size_t *bytes);

/* Attach a KV cache (library housekeeping; no passage of the pages defines it). d_buf == NULL:
 * the library allocates (zeroed) and owns the memory;
 * otherwise d_buf is caller-owned device memory of at least amk_kv_bytes bytes, borrowed
 * until amk_kv_free. max_seq must not exceed the model's max_seq. */
amk_status amk_kv_alloc(amk_model *m, int32_t batch, int32_t max_seq, void *d_buf,
                        size_t buf_bytes, amk_kv **out);

/* Device pointer of the cache (for the caller to prefill or inspect; housekeeping). */
amk_status amk_kv_data(const amk_kv *kv, void **d_ptr);

/* One decode step, asynchronous on `stream`: the decode step of the pages' MegaKernel, all of a
 * token's operators in one persistent launch (Ada-MK technical summary, "Problem Statement" and
 * "Methodology"; greedy decoding as in the AutoMegaKernel abstract). d_tokens: device int32
 * [batch], the token of each
 * sequence at position `pos`. Writes K/V at slot `pos`, attends over [0, pos], writes d_next
 * (device int32 [batch], greedy argmax, lowest index on ties) and, when d_logits != NULL,
 * d_logits (device float32 [batch, vocab]). d_next may alias the next call's d_tokens. Calls on
 * one model must be stream-ordered (scratch is reused). Device-side errors (dependency timeout,
 * token out of range) are recorded on the device and reported by amk_sync. The call may be
 * captured into a graph: the step counter that orders the megakernel's dependency flags lives on
 * the device, so every replay advances it as an eager launch does, and results do not depend on
 * it (a replay gives the eager launch's logits bit for bit). */
amk_status amk_decode_step(amk_model *m, amk_kv *kv, const int32_t *d_tokens, int32_t pos,
                           int32_t batch, float *d_logits, int32_t *d_next, void *stream);

/* n_steps consecutive greedy decode steps in ONE launch (megakernel path): step i runs at position
 * pos + i on the tokens step i-1 produced (step 0 on d_tokens) and writes them to d_out[i][b]
 * (device int32 [n_steps][batch]); d_logits, when not NULL, receives each step's logits
 * (device float32 [n_steps][batch][vocab]). Removes the per-token launch and host round trip:
 * inside the launch a step's first-layer QKV tiles wait for the previous step's argmax, which
 * every task of that step precedes (checked by the schedule validator). The unfused path runs
 * the same steps as consecutive launch sequences. pos + n_steps must not exceed max_seq. Same
 * ordering and error rules as amk_decode_step, which is this call with n_steps = 1. Source: the
 * pages' launch-overhead motivation (Ada-MK summary, "Methodology"). */
amk_status amk_decode_steps(amk_model *m, amk_kv *kv, const int32_t *d_tokens, int32_t pos,
                            int32_t n_steps, int32_t batch, float *d_logits, int32_t *d_out,
                            void *stream);

/* As amk_decode_steps with a position per sequence: h_pos is a HOST array of `batch` positions
 * (read before the call returns), sequence b decodes at h_pos[b] + i in step i, attends over
 * [0, h_pos[b] + i] of its own cache and appends there. Sequences of different lengths share the
 * batched steps, as in the pages' batch sweeps (Ada-MK summary, "Experimental Results", batch
 * sizes 1 to 16). Every h_pos[b] >= 0 and h_pos[b] + n_steps <= max_seq, else AMK_E_CAPACITY. */
amk_status amk_decode_steps_ragged(amk_model *m, amk_kv *kv, const int32_t *d_tokens,
                                   const int32_t *h_pos, int32_t n_steps, int32_t batch,
                                   float *d_logits, int32_t *d_out, void *stream);

/* Capacity (bytes) of the static device array behind amk_decode_steps_noalloc, one per GPU. */
#define AMK_STATIC_SCRATCH_BYTES (64u << 20)

/* amk_decode_steps for callers that cannot allocate device memory: code being captured into a
 * graph, tight serving loops, harnesses that forbid hipMalloc. Same arguments, results and
 * ordering rules as amk_decode_steps (bit for bit the same tokens and logits), but the step's
 * scratch (dependency flags, step counter, activation slots, attention partials, logits when
 * d_logits is NULL) lives in a static device array of AMK_STATIC_SCRATCH_BYTES per GPU, which
 * the library holds until the process ends; the call allocates nothing (no hipMalloc/hipFree).
 * The caller still passes the inputs and outputs. Every call on a GPU, of any model, shares that
 * GPU's array and first clears its flags and step counter, so calls that overlap on one GPU
 * (other streams, other threads) race: serialise them. Errors: AMK_E_CAPACITY when the model's
 * step scratch (amk_model_info.scratch_bytes) exceeds the array; the argument errors of
 * amk_decode_steps. Device-side errors are reported by amk_sync as for the other calls. */
amk_status amk_decode_steps_noalloc(amk_model *m, amk_kv *kv, const int32_t *d_tokens,
                                    int32_t pos, int32_t n_steps, int32_t batch,
                                    float *d_logits, int32_t *d_out, void *stream);

/* Prompt processing: the n_tokens prompt ids d_tokens (device int32 [n_tokens]) of KV sequence
 * `seq` at positions pos0 .. pos0 + n_tokens - 1, run as operator launches whose GEMVs take up to 16
 * tokens at once on the matrix cores (each token a column at its own position, all columns
 * reading and appending the one sequence's KV rows). It writes those KV rows, the greedy next token
 * after the prompt to d_next (device int32 [1]) and, when d_logits is not NULL, the last prompt
 * token's logits (device float32 [vocab]). Decoding then continues at pos0 + n_tokens with
 * amk_decode_step(s). This is the pages' hybrid engine: prompt processing on ordinary fused
 * operators, decoding on the megakernel (Ada-MK summary, "Methodology", Phase II). The first call
 * allocates the scratch of the prompt engine (freed with the model); it is stream-ordered with the
 * model's other calls. Errors: AMK_E_CAPACITY if seq is outside the KV cache or the positions
 * exceed max_seq, AMK_E_INVALID for null pointers or n_tokens < 1. */
amk_status amk_prefill(amk_model *m, amk_kv *kv, int32_t seq, const int32_t *d_tokens,
                       int32_t pos0, int32_t n_tokens, float *d_logits, int32_t *d_next,
                       void *stream);

/* Synchronise `stream` and report a device-side error recorded by earlier steps (and clear it).
 * Housekeeping: the bounded waits behind it make a dependency that never resolves an error
 * instead of a hang. */
amk_status amk_sync(amk_model *m, void *stream);

/* Sizes and the cost-model prediction of the model's schedule (housekeeping). */
amk_status amk_model_get_info(const amk_model *m, amk_model_info *out);

/* Task trace of the megakernel: the profiling behind the offline search (Ada-MK technical summary,
 * "Methodology", Phase I; read by amk_cost_model_fit and amk_schedule_rebalance). d_trace:
 * device buffer of at least
 * 8 * (4 * n_tasks + n_cu) bytes, caller-owned; NULL turns tracing off. While on, every step
 * writes, per task id, four 100 MHz wall-clock stamps (start of wait, wait done, input staged,
 * end) and, after them, the XCC id of each workgroup. Synchronises the device. */
amk_status amk_trace_enable(amk_model *m, uint64_t *d_trace, size_t bytes);

/* Copy of the model's frozen schedule blob, the solidified execution path (Ada-MK technical
 * summary, "Methodology", Phase I) (host memory, release with amk_blob_free). */
amk_status amk_model_get_schedule(const amk_model *m, void **blob, size_t *bytes);

/* Replace the frozen schedule of a megakernel model with another one of the same structure: same
 * config, batch, CU count, task count, KV blocks and LM tiles (e.g. a copy re-tiled by
 * amk_schedule_rebalance). The blob (host) is validated first (AMK_E_SCHEDULE_REJECTED; a
 * different structure gives AMK_E_UNSUPPORTED and leaves the model unchanged). Synchronises
 * `stream`, uploads the task tables and restarts the flag epochs. Not for use while a step of this
 * model is being captured into a graph. */
amk_status amk_model_set_schedule(amk_model *m, const void *blob, size_t bytes, void *stream);

/* Profile-guided tuning of the frozen schedule on the device: the offline search that profiles
 * candidates and solidifies the best path (Ada-MK summary, "Fine-Grained DAG-Based Automatic
 * Search"), applied to the row boundaries of the GEMV tiles. Times `steps` untraced decode steps
 * at positions pos .. pos+steps-1 of `kv` with the current schedule, then `rounds` times: runs
 * those steps with the task trace on, re-tiles the schedule from the traces
 * (amk_schedule_rebalance with `gain`), installs and times it. The fastest schedule measured is
 * kept installed; its mean step time (us) goes to best_us (may be NULL). The steps overwrite
 * those positions' K/V slots of batch row 0..max_batch-1 and use token 0. Allocates a trace buffer
 * for the duration of the call; any trace set by amk_trace_enable is turned off. Megakernel path
 * only (AMK_E_UNSUPPORTED otherwise). Read the result with amk_model_get_schedule and pass it to
 * amk_model_create to reuse it. */
amk_status amk_model_tune(amk_model *m, amk_kv *kv, int32_t pos, int32_t rounds, int32_t steps,
                          double gain, void *stream, double *best_us);

/* Release a KV cache / a model and everything it owns (housekeeping). A caller-owned KV buffer is
 * left alone. Not while a step using them is in flight. */
amk_status amk_kv_free(amk_kv *kv);
amk_status amk_destroy(amk_model *m);

/* Message of the last failure on the calling thread ("" if none). Valid until the next call. */
const char *amk_last_error(void);

/* ---- host-only schedule layer (no GPU needed) ------------------------------------------- */

/* Decompose the decoder into tile tasks, search placement/tiling against `cost` (NULL: default
 * model) and serialise the best schedule for `n_cu` compute units and `batch`. `params` may be
 * NULL. The result (host memory) is released with amk_blob_free. */
amk_status amk_schedule_build(const amk_config *cfg, int32_t batch, int32_t n_cu,
                              const amk_sched_params *params, const amk_cost_model *cost,
                              void **blob, size_t *bytes);

/* Static check of a schedule blob: structure, acyclicity of the dependency graph (with per-CU
 * program order), race freedom and read coverage of every step-local buffer, resource limits.
 * AMK_OK if safe, AMK_E_SCHEDULE_REJECTED otherwise; report (may be NULL) receives a
 * NUL-terminated text of at most report_cap bytes. */
amk_status amk_schedule_validate(const void *blob, size_t bytes, char *report, size_t report_cap);

/* Dynamic cross-check: executes the schedule on the host under several interleavings with
 * monotone flags and shadow memory; reports deadlock or a stale read. Same return convention. */
amk_status amk_schedule_simulate(const void *blob, size_t bytes, char *report, size_t report_cap);

/* Profile-guided re-tiling (host only). traces: n_traces consecutive task traces (each
 * 4 * n_tasks + n_cu uint64 words, as amk_trace_enable writes them for one step) of steps run with
 * this schedule. Within every GEMV phase the row boundaries move a fraction `gain` (0 < gain <= 1)
 * of the way towards those at which the tiles, each starting when it was staged and streaming at
 * its measured rate, would all finish together (the next phase needs all of them). Task ids,
 * placement and waits are kept; attention waits follow the new QKV tiling. The input must
 * validate and so must the result (AMK_E_SCHEDULE_REJECTED). Output in host memory, released with
 * amk_blob_free. */
amk_status amk_schedule_rebalance(const void *blob, size_t bytes, const uint64_t *traces,
                                  int32_t n_traces, double gain, void **out_blob,
                                  size_t *out_bytes);

/* Measure the cost model on the current device (the offline profiling behind the schedule
 * search: Ada-MK technical summary, "Methodology", Phase I, and "Key Contributions" item 2).
 * Microbenchmarks with the megakernel's own device code: the per-CU weight-stream rate with 8,
 * 16, ... and all CUs streaming at once; the time of one dependency hop (wait, stage a vector of
 * K fp32 words, write the next) from one workgroup to the next, for the tagged batch-1 protocol
 * and the flag protocol, within one XCD and across XCDs, with the other CUs idle or streaming;
 * and the all-to-all phase (every CU stages the vector all of them wrote a share of, then writes
 * its share of the next). Fitted: cu_stream_gbs = the all-CU rate per CU; hop_us and l2_gbs from a
 * line through the phases at K = 1024, 4096 and 11008 (time = hop_us + 4 K bytes / l2_gbs);
 * task_us = attn_us = 0 (amk_cost_model_fit reads them off a traced step of the model). report
 * (may be NULL) receives the measurements and the fit as JSON.
 * Allocates about 8 MiB per CU of device memory for the duration of the call; synchronises
 * `stream`; takes a few tenths of a second. */
amk_status amk_calibrate(amk_cost_model *out, char *report, size_t report_cap, void *stream);

/* The cost model the schedule search uses when given none, for n_cu compute units: the
 * calibrated one (see amk_cost_model) or the built-in values. source (may be NULL) receives the
 * path of the file it came from, or "built-in". Host only. */
amk_status amk_cost_model_default(int32_t n_cu, amk_cost_model *out, char *source,
                                  size_t source_cap);

/* Cost-model makespan (us) of a schedule at context length ctx. */
amk_status amk_schedule_predict(const void *blob, size_t bytes, const amk_cost_model *cost,
                                int32_t ctx, double *makespan_us);

/* The cost model's timeline of one step of a schedule at context length ctx, written as the task
 * trace amk_trace_enable records (trace_words >= 4 * n_tasks + n_cu): per task, 100 MHz stamps
 * of when its CU picks it up (twice), when its input is staged (an attention block: when its
 * partial is done) and when it finishes; then n_cu zero words. A predicted step can so be
 * exported and compared like a measured one. Host only; AMK_E_INVALID on a malformed blob or a
 * short buffer. */
amk_status amk_schedule_predict_trace(const void *blob, size_t bytes, const amk_cost_model *cost,
                                      int32_t ctx, uint64_t *trace, size_t trace_words);

/* Fit a cost model's fixed costs to measured task traces of one schedule (the per-model offline
 * profiling of Ada-MK technical summary, "Methodology", Phase I): n_traces consecutive traces as
 * amk_trace_enable writes them, of steps at context length ctx. Rates and prefetch come from
 * `base` (zero fields: the default model, e.g. amk_calibrate's); hop_us, task_us and attn_us are
 * the medians of what the traced tasks took beyond the simulation's other terms (hop: tiles that
 * waited, staged time less staging and the last producer's end; task: GEMV tiles' end beyond
 * their streaming; attn: attention partials' end beyond their staging and streaming). report
 * (may be NULL) receives JSON with the sample counts, the measured and predicted step (us) and
 * the fitted model in the "fit" object, in the format cost_model.json uses. Host only. */
amk_status amk_cost_model_fit(const void *blob, size_t bytes, const uint64_t *traces,
                              int32_t n_traces, int32_t ctx, const amk_cost_model *base,
                              amk_cost_model *out, char *report, size_t report_cap);

void amk_blob_free(void *blob);

#ifdef __cplusplus
}
#endif

#endif /* AMK_H */
