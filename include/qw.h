/*
 * qw.h -- C ABI of libqw.so: the Qwen2 decoder forward pass (prefill and
 * KV-cached greedy decode) on one AMD Instinct MI355X (gfx950).
 *
 * The operation is the one the pages describe:
 *   - "augur" (feature list): RMSNorm before attention, before the MLP and
 *     after the last layer; RoPE on q and k; grouped-query attention; causal
 *     masking; SwiGLU MLP; pre-norm decoder blocks; embeddings -> layers ->
 *     final norm -> LM head; greedy generation; a prefill/decode split; a
 *     preallocated KV cache.
 *   - "LLM Speedrun: Architecture": sections "Attention", "Every token with
 *     every other token", "Grouped Query Attention GQA", "Rotary Positional
 *     Embeddings RoPE", "Split-half RoPE implementation", "Introducing bias",
 *     "Decoding"; its harness listing fixes weight layouts ([out, in]) and the
 *     generation loop (the prompt once, then one token per step).
 *   - "Building a Qwen2.5-1.5B Inference Engine From Scratch", section 1:
 *     prefill processes every prompt token at once and fills the KV cache;
 *     decode then feeds one new token per sequence per step.
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers (hipMalloc'd or torch CUDA tensors
 *     on the current device) unless a comment says "host".
 *   - All work is enqueued on the hipStream_t given to qw_create (0 = the
 *     legacy default stream).  Outputs are valid once the caller synchronises
 *     that stream.  qw_prefill and qw_decode_step do not wait for the GPU
 *     and make no device allocation of their own (qw_decode_step captures
 *     and instantiates a HIP graph on its first call for a batch size and
 *     context range); qw_create waits for its own set-up work, and
 *     qw_destroy and the check and timing helpers synchronise the stream.
 *   - Every call returns a qw_status.  On anything but QW_OK, qw_last_error()
 *     returns a message for the calling thread; argument and state errors
 *     are detected on the host before anything is enqueued, so the model is
 *     unchanged.
 *   - One qw_model must not be used from two host threads at once.
 */
#ifndef QW_H_
#define QW_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qw_status {
  QW_OK = 0,
  QW_ERR_INVALID_ARG = -1,    /* bad pointer, shape, or config value          */
  QW_ERR_OUT_OF_MEMORY = -2,  /* a device allocation failed                    */
  QW_ERR_HIP = -3,            /* a HIP runtime call failed (message has it)    */
  QW_ERR_CACHE_FULL = -4,     /* the step would write past max_seq             */
  QW_ERR_BAD_STATE = -5,      /* e.g. decode before any prefill                */
  QW_ERR_UNSUPPORTED = -6,    /* valid model, but a shape no kernel covers     */
  QW_ERR_NUMERICS = -7        /* qw_check_numerics: a value left its range     */
} qw_status;

/* Storage type of every weight tensor handed to qw_create.
 *   QW_F32 : float32 weights; the whole forward runs in fp32 arithmetic.
 *   QW_BF16: bf16 weights.  GEMM operands (weights and activations) are held
 *            in fp16 with fp32 accumulation; the residual stream, softmax,
 *            norms' statistics and logits are fp32.  Each weight group
 *            (a layer's q/k/v, o, gate/up, down; the embedding; the LM head)
 *            is multiplied by a power of two 2^k that puts its largest
 *            magnitude A in [2^14, 2^15) and rounded to fp16, which the
 *            kernels undo exactly.  A value v converts without rounding when
 *            |v| >= A * 2^-32 (bf16's 8 significant bits still fit fp16's
 *            normal or subnormal spacing); a smaller v is rounded with an
 *            absolute error below A * 2^-39.  Activations held in fp16 must
 *            stay below 65504 in magnitude: qw_check_numerics reports a
 *            forward that left that range (it surfaces as an inf or NaN
 *            logit) or the decode residual's fixed-point range.
 *   QW_F16 : fp16 weights ("Building a Qwen2.5-1.5B Inference Engine From
 *            Scratch", section 1.1: FP16 as the next experiment after FP32);
 *            the same arithmetic as QW_BF16, the weights scaled the same way
 *            (exact while |v| >= A * 2^-32 as above). */
typedef enum qw_dtype { QW_F32 = 0, QW_BF16 = 1, QW_F16 = 2 } qw_dtype;

/* Model and capacity.  Field meanings follow the Qwen2 config names the
 * "augur" feature list enumerates. */
typedef struct qw_config {
  int32_t n_layers;       /* decoder blocks                                   */
  int32_t hidden;         /* H, model width                                   */
  int32_t n_heads;        /* query heads nq                                   */
  int32_t n_kv_heads;     /* KV heads nkv; nq % nkv == 0 (GQA)                */
  int32_t head_dim;       /* hd; 32, 64 or 128 (the kernels' head sizes)      */
  int32_t intermediate;   /* I, SwiGLU width                                  */
  int32_t vocab;          /* V                                                */
  float rms_eps;          /* RMSNorm epsilon (1e-6 for Qwen2.5)               */
  float rope_theta;       /* RoPE base (1e6 for Qwen2.5)                      */
  int32_t qkv_bias;       /* must be 1: q/k/v projections carry a bias        */
  int32_t tie_embeddings; /* 1: LM head = embedding; 0: weights.lm_head used  */
  qw_dtype dtype;         /* storage type of all weight tensors               */
  int32_t max_batch;      /* largest batch any later call may use             */
  int32_t max_seq;        /* KV-cache positions per sequence                  */
} qw_config;

/* One decoder block's tensors, HF layouts: projection weights are row-major
 * [out, in]; vectors are [n].  Every pointer is a device pointer of `dtype`. */
typedef struct qw_layer_weights {
  const void *input_norm;     /* [H]                                          */
  const void *q_w, *q_b;      /* [nq*hd, H], [nq*hd]                           */
  const void *k_w, *k_b;      /* [nkv*hd, H], [nkv*hd]                         */
  const void *v_w, *v_b;      /* [nkv*hd, H], [nkv*hd]                         */
  const void *o_w;            /* [H, nq*hd]   (no bias)                        */
  const void *post_norm;      /* [H]                                          */
  const void *gate_w, *up_w;  /* [I, H]       (no bias)                        */
  const void *down_w;         /* [H, I]       (no bias)                        */
} qw_layer_weights;

typedef struct qw_weights {
  const void *embed;                /* [V, H] token embedding                  */
  const void *final_norm;           /* [H]                                     */
  const void *lm_head;              /* [V, H], or NULL when tie_embeddings     */
  const qw_layer_weights *layers;   /* HOST array of n_layers entries          */
} qw_weights;

typedef struct qw_model qw_model;

/* Build a model on the current HIP device.
 * Reads every weight once to make the library's own packed copies (fused QKV
 * with fp32 bias, row-interleaved gate/up, fp16 or fp32 compute copies; in
 * fp16 mode also, wherever the prefill or decode kernels read it (always
 * for hidden <= 4096), a second copy of every projection and of the LM head
 * in the kernels' tiled operand order: about twice the weight bytes), so the
 * caller's weight buffers may be freed after this returns.  Allocates the
 * KV cache (2 * n_layers * max_batch * nkv * max_seq * hd elements of the
 * compute type), a RoPE cos/sin table for max_seq positions, and workspace for
 * max_batch * max_seq prefill rows (including the split-K slices of every
 * GEMM shape a later call can reach, so prefill and decode never allocate).
 * `hip_stream` (a hipStream_t) is the stream all later work is enqueued on.
 * Waits for its set-up work.
 * Errors: INVALID_ARG (NULL pointers, non-positive sizes, nq % nkv != 0, odd
 * head_dim, qkv_bias != 1, lm_head NULL while untied), UNSUPPORTED (head_dim
 * not in {32, 64, 128}, hidden or intermediate not a multiple of 64, an inf
 * or NaN projection or embedding weight in bf16 mode), OUT_OF_MEMORY, HIP.
 * On error *out is set to NULL.
 * Source: "augur" (preallocated KV cache); "LLM Speedrun: Architecture",
 * harness listing (weight names and [out, in] layouts). */
qw_status qw_create(const qw_config *cfg, const qw_weights *weights, void *hip_stream,
                    qw_model **out);

/* Paged KV cache ("augur", "Not yet" list: paged attention).  The same model
 * as qw_create, but each layer's cache is a pool of `num_blocks` blocks of
 * QW_KV_BLOCK positions (2 * n_layers * num_blocks * nkv * QW_KV_BLOCK * hd
 * elements of the compute type in all), and every sequence holds a table of
 * the blocks its positions live in, so the pool is sized for the positions
 * actually held rather than max_batch * max_seq.  The library owns the pool:
 * a prefill (qw_prefill, qw_prefill_ragged, qw_generate) returns every block
 * to it and gives each sequence the blocks of its prompt; a decode step gives
 * a sequence one more block each time its new token starts one.  max_seq
 * still bounds each sequence and sizes the RoPE table and the block tables.
 * All other calls behave as on a dense model, with the same results bit for
 * bit (the kernels do the same arithmetic; only addresses differ).
 * Errors: as qw_create; INVALID_ARG (num_blocks < 1). */
#define QW_KV_BLOCK 64
qw_status qw_create_paged(const qw_config *cfg, const qw_weights *weights, int32_t num_blocks, void *hip_stream,
                          qw_model **out);

/* Prefill: run `batch` equal-length prompts ids[batch][prompt_len] (int32,
 * device, each in [0, V)) through the model at positions 0 .. prompt_len-1,
 * writing their keys and values into the cache.  Every sequence restarts at
 * position 0 (earlier cache contents are overwritten).
 * Outputs (device):
 *   next_ids[batch]    greedy token of each sequence: the lowest index of the
 *                      largest logit of its last prompt position.
 *   logits             NULL, or fp32 [batch][V] for each last position, or,
 *                      when logits_all != 0, fp32 [batch][prompt_len][V] for
 *                      every position (meant for checks on small models).
 * Token ids outside [0, V) are read as id 0 (never out of bounds) and make
 * qw_check_ids report an error.
 * Errors: INVALID_ARG (NULL ids/next_ids, batch < 1 or > max_batch,
 * prompt_len < 1), CACHE_FULL (prompt_len > max_seq), HIP.
 * Source: "Building a Qwen2.5-1.5B Inference Engine From Scratch", section 1
 * (prefill runs the whole prompt at once and fills the KV cache); "augur"
 * (causal masking, greedy generation, lowest index among equal maxima read
 * from the harness listing's argmax). */
qw_status qw_prefill(qw_model *m, const int32_t *ids, int32_t batch, int32_t prompt_len,
                     float *logits, int32_t logits_all, int32_t *next_ids);

/* Ragged prefill ("augur", "Not yet" list: batching of prompts of different
 * lengths): n_seqs prompts of lens[b] tokens (lens: HOST array, each in
 * [1, max_seq]) packed back to back in ids[sum(lens)] (device), no padding.
 * Sequence b goes to batch row b at positions 0 .. lens[b] - 1; every row
 * attends causally within its own sequence only.  Outputs as qw_prefill
 * without logits_all: next_ids[n_seqs]; logits NULL or fp32 [n_seqs][V] of
 * each sequence's last position.  Later qw_decode_step calls continue every
 * sequence from its own position.  Works on dense and paged models.
 * Errors: INVALID_ARG (NULL pointers, n_seqs outside [1, max_batch], a length
 * < 1), CACHE_FULL (a length > max_seq, or a paged pool too small for the
 * prompts), HIP. */
qw_status qw_prefill_ragged(qw_model *m, const int32_t *ids, const int32_t *lens, int32_t n_seqs, float *logits,
                            int32_t *next_ids);

/* One greedy decode step for every sequence of the last prefill: feeds
 * ids[batch] (device; may alias the previous call's next_ids) at each
 * sequence's next position (its own after a ragged prefill), appends their
 * keys and values to the cache, and writes next_ids[batch] and, if non-NULL,
 * fp32 logits[batch][V].  Positions advance on the device, so steps may be
 * enqueued back to back without host syncs.
 * Errors: INVALID_ARG (NULL ids/next_ids), BAD_STATE (no prefill yet),
 * CACHE_FULL (a sequence already holds max_seq positions, or a paged pool has
 * no free block for a sequence that needs one), HIP.
 * Source: "Building a Qwen2.5-1.5B Inference Engine From Scratch", section 1
 * (decode feeds one new token per step against the cache); "LLM Speedrun:
 * Architecture", "Decoding" and the harness listing's generation loop. */
qw_status qw_decode_step(qw_model *m, const int32_t *ids, float *logits, int32_t *next_ids);

/* Greedy generation of `steps` tokens after `batch` equal-length prompts
 * ids[batch][prompt_len] (device), all enqueued on the model's stream without
 * host synchronisation: the pages' generation loop (the prompt once, then one
 * token per step: "LLM Speedrun: Architecture", harness listing; "augur",
 * greedy generation and cache benchmarking; "Building a Qwen2.5-1.5B
 * Inference Engine From Scratch", section 1.1, use_cache=False as ground
 * truth).
 *   use_cache != 0: qw_prefill, then `steps` KV-cached decode steps.
 *   use_cache == 0: step k (0 .. steps) runs a prefill over the prompt and
 *     the k tokens generated so far (positions 0 .. prompt_len + k - 1) and
 *     takes the greedy token of its last row; no step reuses keys or values
 *     an earlier step computed.
 * Outputs (device): out_ids [batch][steps + 1] (the prefill's token, then one
 * per step); logits NULL or fp32 [batch][steps + 1][V].  Afterwards the model
 * holds the sequences' cache (positions 0 .. prompt_len + steps - 1), so
 * qw_decode_step may continue them.
 * Errors: INVALID_ARG (NULL ids/out_ids, batch outside [1, max_batch],
 * prompt_len < 1, steps < 0), CACHE_FULL (prompt_len + steps > max_seq),
 * HIP. */
qw_status qw_generate(qw_model *m, const int32_t *ids, int32_t batch, int32_t prompt_len, int32_t steps,
                      int32_t use_cache, int32_t *out_ids, float *logits);

/* Size of the static device array behind qw_decode_step_noalloc (per GPU). */
#define QW_NOALLOC_SCRATCH_BYTES (16u << 20)

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * decode step as qw_decode_step (same kernels, same results, bit for bit),
 * launched one kernel at a time on the model's stream (nothing is captured
 * or instantiated, no event created), with every per-step buffer (the
 * fixed-point residual and projection sums, split-KV partials, LM-head argmax
 * partials, f16 activations) in one static device array of
 * QW_NOALLOC_SCRATCH_BYTES that the library holds on each GPU until the
 * process ends.  logits (fp32 [batch][V], device, or NULL) and next_ids
 * [batch] are written directly.  The step's kernels clear what they
 * accumulate into, so stale contents of the array do not matter; but every
 * call on one GPU (any model) shares the array, so calls that overlap on one
 * GPU race: the caller serialises them.  The model's device must be current.
 * Errors: as qw_decode_step; UNSUPPORTED when the model takes the generic
 * step (fp32 weights, max_batch > 32, more than 8 query heads per KV head)
 * or the step's buffers exceed QW_NOALLOC_SCRATCH_BYTES (about 7 MB at
 * batch 32 of the 1.5B shapes); BAD_STATE when another device is current. */
qw_status qw_decode_step_noalloc(qw_model *m, const int32_t *ids, float *logits, int32_t *next_ids);

/* Free everything the model owns.  Synchronises its stream first.  NULL is a
 * no-op.  Source: "augur" (the preallocated cache lives as long as the model). */
qw_status qw_destroy(qw_model *m);

/* Message of the calling thread's last error ("" if none).  The pointer stays
 * valid until that thread's next qw_* call. */
const char *qw_last_error(void);

/* ---- inspection and measurement helpers (not on the hot path) ----------- */

/* Host view of the state: *batch of the last prefill (0 if none) and *pos,
 * the number of cache positions the longest sequence holds. */
qw_status qw_get_state(const qw_model *m, int32_t *batch, int32_t *pos);

/* Cache positions held by each of the first n sequences, into the HOST array
 * pos[n] (0 past the batch).  No synchronisation: host bookkeeping.
 * Errors: INVALID_ARG (NULL, n outside [0, max_batch]). */
qw_status qw_get_positions(const qw_model *m, int32_t *pos, int32_t n);

/* Paged models: free and total blocks of the pool (HOST outputs); 0 and 0 on
 * a dense model.  Errors: INVALID_ARG (NULL). */
qw_status qw_kv_blocks(const qw_model *m, int32_t *free_blocks, int32_t *total_blocks);

/* Synchronise the stream and report whether any token id handed to prefill or
 * decode since the last check was outside [0, V): QW_ERR_INVALID_ARG if so
 * (and the flag is cleared), QW_OK otherwise. */
qw_status qw_check_ids(qw_model *m);

/* Synchronise the stream and report whether, since the last check, a logit
 * of a greedy row was inf or NaN (an fp16 activation overflowed, or a weight
 * was non-finite) or an addend of the decode step's fixed-point residual or
 * projection sums exceeded 2^23 in magnitude (it was clamped):
 * QW_ERR_NUMERICS if so (those flags are cleared), QW_OK otherwise. */
qw_status qw_check_numerics(qw_model *m);

/* Sampling instead of the greedy choice for every later prefill, decode step
 * and generation ("augur": temperature, top-k and top-p sampling).  The pages
 * give no formulas, so the plain reading is used: keep the top_k largest
 * logits (ties: lower index first), weight them by exp((l - l_max) /
 * temperature), keep the shortest prefix of that order whose cumulative
 * weight reaches top_p of their total, and pick the first kept token whose
 * cumulative weight exceeds u times the kept total.  u in [0, 1) is the top
 * 24 bits of the first word of Philox-4x64-10 (Salmon et al., SC 2011) at
 * counter (n, b, 0, 0) and key (seed, 0), where b is the batch row and n the
 * number of tokens the sequence holds before the chosen one; so the draws
 * depend only on (seed, row, position), with or without the cache.
 * Arguments: temperature > 0, 1 <= top_k <= 1024, 0 < top_p <= 1;
 * top_k = 0 restores the greedy choice.  Errors: INVALID_ARG. */
qw_status qw_set_sampling(qw_model *m, float temperature, int32_t top_k, float top_p, uint64_t seed);

/* End of sequence ("augur": EOS stopping; the speedrun harness stops on the
 * end-of-stream token): with eos_id >= 0, a sequence that emits eos_id is
 * finished, and every later prefill-free step emits eos_id for it again, on
 * the device, inside the decode step (no host round trip).  Each qw_prefill
 * (and qw_generate) starts its sequences unfinished.  eos_id = -1 turns the
 * rule off.  Errors: INVALID_ARG (eos_id outside [-1, V)). */
qw_status qw_set_eos(qw_model *m, int32_t eos_id);

/* Synchronise the stream and copy the finished flags of the first n
 * sequences (0 or 1) to the HOST array finished[n] (all 0 while no eos is
 * set).  Errors: INVALID_ARG (NULL, n outside [0, max_batch]), HIP. */
qw_status qw_get_finished(qw_model *m, int32_t *finished, int32_t n);

/* Decode-step execution: 1 (default) replays a captured HIP graph of the whole
 * step; 0 launches its kernels one by one.  Both run the same kernels on the
 * same data and give identical results. */
qw_status qw_set_graph(qw_model *m, int32_t enable);

/* Kernel timing for roofline reports.  While enabled, decode steps run
 * without the graph and every launch of the kernel family `name` (see
 * qw_kernel_names) is bracketed by hipEvents on the model's stream; the
 * elapsed times accumulate.  qw_timing_read synchronises the stream and
 * returns the total milliseconds and launch count since the last reset. */
qw_status qw_timing_enable(qw_model *m, const char *name);
qw_status qw_timing_read(qw_model *m, double *total_ms, int64_t *launches, int32_t reset);

/* Comma-separated names of the kernel families the library launches. */
const char *qw_kernel_names(void);

/* Measured peaks, the denominators a run can reach beside the published
 * ones (not on the forward pass).  Both enqueue on `hip_stream`, wait for
 * their own work, and report through qw_last_error.
 * qw_peak_copy: `iters` passes of a 16-byte-per-lane grid-stride kernel
 *   over `bytes` (a positive multiple of 64 MiB) of src (device pointers,
 *   src and dst not overlapping, dst as large as src).  read_only = 0: dst
 *   = src, *gbs = (bytes read + bytes written) / seconds / 1e9.  read_only
 *   = 1: every byte of src is read once per pass and at most 16 MiB of dst
 *   written (one combination of its reads per thread); the pass runs with
 *   two load layouts at 4, 8 and 16 workgroups per CU and *gbs is the best
 *   bytes read / seconds / 1e9 (the pattern of the decode step, which reads
 *   far more than it writes).
 * qw_peak_mfma: 8192 waves each issue `iters` rounds of eight independent
 *   16x16x32 fp16 matrix products (v_mfma_f32_16x16x32_f16) on register
 *   operands; *tflops = dense fp16 FLOP / seconds / 1e12.
 * Errors: INVALID_ARG (NULL output or pointers, bad sizes), HIP. */
qw_status qw_peak_copy(void *dst, const void *src, int64_t bytes, int32_t iters, int32_t read_only,
                       void *hip_stream, double *gbs);
qw_status qw_peak_mfma(int32_t iters, void *hip_stream, double *tflops);

#ifdef __cplusplus
}
#endif

#endif /* QW_H_ */
