/*
 * rlt.h - C ABI of the Recurrent Looped Transformer transition library (MI355X / gfx950).
 *
 * The library computes the method's forward pass on one GPU: the token-parallel
 * causal encoder and its memory projection, the per-token decoder transition
 * u_t = Merge(e_t, s_{t-1}), H_t = D_phi(u_t; M_<=t, C^D_{t-1}, t) batched over
 * independent sequences, the RLT-2 chunked-feedback and RLT-0 variants, and the
 * readout.  Sources (web pages about the method):
 *   [S] greeksharifa.github.io, "Recurrent Looped Transformer 요약 설명":
 *       §2.1-§2.7 (state, encoder/memory, transition, prefill/decoding, merge,
 *       blocks, RLT-0/1/2), appendix A.1 (sharing), E (multi-turn), F
 *       (execution procedures F.1 prefill, F.2 generation, F.4 replay), I (RLT-2).
 *   [R] jiphyeonjeon.kr/blog/rlt, "Recurrent Looped Transformer":
 *       §2 eq 2.1-2.2 (memory), §3.1 eq 2.7 (composition), §3.2 (E^step),
 *       §3.3 eq 2.9-2.16 (merge, blocks, window), §4.2 eq 3.3 (storage),
 *       §6.2 eq 5.5 (replay log-probabilities), §6.4-6.5 (stale caches, replay).
 *
 * Conventions
 *  - Every function returns an rlt_status (0 = RLT_OK). No C++ exception crosses
 *    the boundary. rlt_last_error() returns a thread-local message for the last
 *    failure in the calling thread.
 *  - Pointers marked "device" are HIP device memory on the model's device; the
 *    caller owns them. The library owns the packed weights and all state
 *    buffers (decoder state, rings, memory, encoder cache, workspaces).
 *  - Calls enqueue work on the given stream and return without synchronising,
 *    except rlt_create / rlt_update_weights / rlt_state_create, which
 *    synchronise the stream before returning.
 *  - Host-side validation (shapes, capacity, configuration, staleness) runs
 *    before any launch; on error nothing is enqueued and the state is unchanged.
 *  - Token ids must lie in [0, vocab); other ids are undefined behaviour.
 *  - Batches are rectangular: every row of a state is at the same position.
 *  - Positions are 1-based; position 1 holds BOS. Chunks of RLT-2 are anchored
 *    at position 1 ([S] appendix I.1).
 *  - A state is bound to the model that created it; it is stale after
 *    rlt_update_weights until rlt_state_reset ([R] §6.4: caches computed with
 *    old parameters are not current-policy values).
 */
#ifndef RLT_H
#define RLT_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RLT_OK = 0,
  RLT_ERR_INVALID_ARG = -1,   /* null pointer, bad size, inconsistent config, unknown weight name */
  RLT_ERR_UNSUPPORTED = -2,   /* a form the pages do not define (e.g. G not in {1, L_D}) or not built */
  RLT_ERR_OOM = -3,           /* device allocation failed */
  RLT_ERR_CAPACITY = -4,      /* positions would exceed the state's max_len */
  RLT_ERR_STALE_STATE = -5,   /* state built under older weights; reset it */
  RLT_ERR_HIP = -6,           /* a HIP runtime call failed */
  RLT_ERR_ORDER = -7          /* decoder asked to consume positions not yet encoded */
} rlt_status;

/* Arithmetic type of the path. RLT_BF16 / RLT_FP16: the 16-bit storage and MFMA input type
 * (weights are rounded to it on create; fp16 keeps 11 significant bits, so weights that are
 * bf16 values stay exact unless their magnitude is below 2^-14, where fp16 spacing 2^-24 applies).
 * RLT_FP16X2: fp16 weights, caches and memory, with every GEMM activation input carried as two
 * fp16 terms (hi + lo, about 22 significant bits) and multiplied as two MFMA products; for the
 * deepest shapes, where one 16-bit rounding per sublayer input adds up past the logit tolerance. */
typedef enum { RLT_FP32 = 0, RLT_BF16 = 1, RLT_FP16 = 2, RLT_FP16X2 = 3 } rlt_dtype;
typedef enum { RLT_V0 = 0, RLT_V1 = 1, RLT_V2 = 2 } rlt_variant;

/* Model configuration ([S] §2.1-§2.7, §3.1; [R] §2-§3). Plain old data. */
typedef struct {
  int vocab;          /* V */
  int d;              /* residual width d (encoder output and recurrent output) */
  int n_heads;        /* H: heads of every attention (encoder, SWA, cross) */
  int d_head;         /* dh (even) */
  int L_E;            /* encoder blocks */
  int L_D;            /* decoder blocks (0 allowed: the model is the gated recurrence) */
  int ffn;            /* SwiGLU hidden width f */
  int window;         /* SWA window W >= 1, counting the current token */
  int groups;         /* memory groups G: 1 (shared) or L_D (one per decoder layer) */
  rlt_variant variant;/* RLT-0 (no feedback), RLT-1 (every token), RLT-2 (chunked) */
  int chunk;          /* RLT-2 feedback interval K_c >= 1 (must be 1 unless RLT-2) */
  int share_enc_dec;  /* 1: decoder SWA Q/K/V/O and FFN alias encoder layer l ([S] appendix A.1); needs L_E == L_D */
  rlt_dtype dtype;    /* storage of matrices, GEMM inputs, K/V, rings and memory; accumulation,
                         residual stream, s, norms, softmax and logits are fp32 */
  float alpha;        /* feedback scale (0.1 in the pages' experiments) */
  float rms_eps;      /* RMSNorm epsilon (1e-6) */
  float rope_base;    /* rotary base (10000) */
} rlt_config;

/* One parameter tensor: fp32 values, row-major, in DEVICE memory, named as in the
 * manifest (emb, enc.{l}.{n1,wq,wk,wv,wo,n2,w1,w3,w2}, mem.nE, mem.{g}.{wk,wv},
 * merge.{ns,wg,bg,ws,s0}, dec.{l}.{m1,wq,wk,wv,wo,m2,xq,xo,m3,w1,w3,w2}, out.{nO,w});
 * matrices are [out_features, in_features]; merge.wg is [d, 2d] over [e_t ; r].
 * numel must match the configuration's shape for that name. */
typedef struct {
  const char* name;
  const float* data;
  int64_t numel;
} rlt_tensor;

typedef struct rlt_model rlt_model;
typedef struct rlt_state rlt_state;

/* Load the parameters theta that every procedure of [S] appendix F runs with (F.1
 * prefill, F.2 generation, F.4 replay all take the current weights as given; [R] §6.4:
 * replay uses the current parameters). Validate cfg, allocate library-owned packed
 * weights on the current device and copy/convert the given tensors into them (the
 * caller may free its tensors once this returns). Every manifest name for cfg must be present exactly once.
 * Errors: INVALID_ARG (bad config / missing or mis-sized tensor), UNSUPPORTED
 * (G not in {1, L_D}, d_head odd, share with L_E != L_D), OOM, HIP. */
int rlt_create(const rlt_config* cfg, const rlt_tensor* weights, int n_weights,
               hipStream_t stream, rlt_model** out);

/* Replace the parameter values (same names and sizes as rlt_create). Every state
 * created before becomes stale ([R] §6.4) until rlt_state_reset. */
int rlt_update_weights(rlt_model* m, const rlt_tensor* weights, int n_weights, hipStream_t stream);

/* Free the model. States of this model must be destroyed first: every cache a state holds
 * was computed with these parameters and means nothing under others ([R] §6.4: caches
 * built with old parameters are stale). Errors: INVALID_ARG (null, or states remain). */
int rlt_destroy(rlt_model* m);

/* Allocate a batch state for `batch` sequences of up to `max_len` positions: the
 * recurrent output s (and RLT-2 register), the per-layer SWA rings C^D, the
 * encoder memory M^g_<=t, the encoder outputs, and (keep_encoder_cache != 0) the
 * per-layer encoder cache C^E needed to encode further tokens after the first
 * encode call (generation, multi-turn appends; [S] §2.4, appendix E). The state
 * starts at H_0 = (s*, empty) ([R] §3.1). Errors: INVALID_ARG, OOM, HIP. */
int rlt_state_create(rlt_model* m, int batch, int max_len, int keep_encoder_cache,
                     hipStream_t stream, rlt_state** out);

/* H_0 = (s*, empty caches), positions reset to 0; clears staleness. */
int rlt_state_reset(rlt_model* m, rlt_state* s, hipStream_t stream);

/* Free a state: its encoder cache, memory, rings and s. The pages' procedures end a
 * sequence's use of its state here ([S] appendix F.2 generation ends; [R] §6.4: after a
 * parameter update cached states are invalidated, not reused). Errors: INVALID_ARG. */
int rlt_state_destroy(rlt_state* s);

/* Bytes of device memory held by the state, split as in [R] §4.2 eq 3.3:
 * out[0] encoder cache C^E, out[1] memory M, out[2] decoder rings C^D,
 * out[3] recurrent output and register, out[4] encoder outputs / gate inputs,
 * out[5] workspaces. Any pointer may be null. */
int rlt_state_bytes(const rlt_state* s, int64_t out[6]);

/* Positions encoded so far and positions consumed by the decoder. */
int rlt_state_positions(const rlt_state* s, int* n_encoded, int* n_decoded);

/* Token-parallel causal encoding of positions n_enc+1 .. n_enc+T for every row
 * ([S] §2.2, §2.4, appendix F.1): e_t, the memory entries of every group
 * (k^g_t = RoPE_t(W^g_K RMSNorm_E(e_t)), v^g_t = W^g_V RMSNorm_E(e_t), [R] eq 2.1-2.2),
 * and C^E when kept. Does not advance the decoder.
 * tokens: device int32 [B, T] row-major. Errors: CAPACITY (n_enc + T > max_len),
 * UNSUPPORTED (n_enc > 0 without an encoder cache), STALE_STATE, INVALID_ARG. */
int rlt_encode(rlt_model* m, rlt_state* s, const int32_t* tokens, int T, hipStream_t stream);

/* Consume the next T encoded positions in order, one transition each
 * ([S] §2.3-§2.7; [R] §3.1 eq 2.7, §3.3 eq 2.9-2.16). RLT-2 runs each chunk's
 * positions together inside every layer; RLT-0 runs positions in parallel.
 * Outputs (device, each nullable):
 *   logits       fp32 [B, T, V]   logits_t = W_out RMSNorm_out(s_t), predicting x_{t+1}
 *   next_logprob fp32 [B, T]      log softmax(logits_t)[next_tokens[b, t]] ([R] eq 5.5)
 *   next_tokens  int32 [B, T]     required when next_logprob is given; an entry < 0 writes 0
 *   s_out        fp32 [B, T, d]   s_t
 * Errors: ORDER (n_dec + T > n_enc), STALE_STATE, INVALID_ARG. */
int rlt_decode_scan(rlt_model* m, rlt_state* s, int T, float* logits, float* next_logprob,
                    const int32_t* next_tokens, float* s_out, hipStream_t stream);

/* Generation step F.2 ([S] §2.4, appendix F.2; [R] §3.2): consume x_t for every row
 * (encoder step with C^E, memory append, one transition) and write the fp32 logits
 * [B, V] that predict x_{t+1}. tokens: device int32 [B]. Needs keep_encoder_cache
 * unless the state is at position 0. Errors as rlt_encode. */
int rlt_step(rlt_model* m, rlt_state* s, const int32_t* tokens, float* logits, hipStream_t stream);

/* Current-policy replay F.4 ([R] §6.2 eq 5.5, §6.5; [S] §2.8): from a fresh H_0 with
 * the current weights, encode tokens [B, T] (x_1 = BOS), rebuild s_t, every SWA
 * ring and the memory, and write logprob[b, t-1] = log p(x_{t+1} | x_<=t) for
 * t = 1..T-1 (fp32 [B, T-1], device). s_out (nullable) receives s_t fp32 [B, T, d].
 * `state` must have batch B and max_len >= T; it is reset first and holds H_T after. */
int rlt_replay(rlt_model* m, rlt_state* state, const int32_t* tokens, int T, float* logprob,
               float* s_out, hipStream_t stream);

/* Exact prefix snapshot ([R] §6.5 and [S] appendix E: an exact prefix checkpoint holds the
 * encoder cache, the encoder-derived cross-attention memory, the complete decoder state,
 * the token and position metadata, the SWA window convention and the model version).
 * The payload (opaque bytes) holds s, the RLT-2 register, every decoder ring C^D, the memory
 * prefix M_<=n_encoded of every group, the encoder cache prefix when the state keeps it, and
 * the encoder outputs of encoded positions not yet consumed; the info block holds the
 * positions, the dependent block-step count, the ring layout (window, ring slots) and two
 * digests: of the configuration, and of the packed parameter values (the model version: a
 * snapshot is valid for any model with the same configuration and parameter values, in this
 * process or another). Restoring then continuing with the same calls gives bit-identical
 * results to never having stopped (serving-split invariance, [R] Proposition 3.1). A prefix
 * edit (deleting, rewriting or truncating earlier tokens) is served by restoring an earlier
 * snapshot that precedes the edit and encoding the new tokens from there ([R] §6.5: a state
 * that contains removed content must not be kept). */
typedef struct {
  uint64_t config_digest;   /* configuration fields */
  uint64_t weights_digest;  /* packed parameter values */
  int32_t batch;
  int32_t n_encoded;        /* positions encoded (memory and encoder-cache prefix length) */
  int32_t n_decoded;        /* positions consumed by the decoder */
  int32_t window;           /* W */
  int32_t ring_slots;       /* slots per ring (W + positions per pass - 1) */
  int32_t has_encoder_cache;
  int64_t block_steps;      /* dependent decoder block passes so far */
  int64_t bytes;            /* payload bytes */
} rlt_snapshot_info;

/* Payload bytes rlt_snapshot needs for the state as it stands. Errors: STALE_STATE, INVALID_ARG. */
int rlt_snapshot_size(rlt_model* m, rlt_state* s, int64_t* bytes);

/* Copy the state's prefix into dst (device memory, or host memory: pinned host memory keeps the
 * call asynchronous) and fill *info on the host. dst must hold rlt_snapshot_size bytes
 * (`capacity`); it is written when the stream reaches the copies. Errors: CAPACITY (dst too
 * small), STALE_STATE, INVALID_ARG. */
int rlt_snapshot(rlt_model* m, rlt_state* s, void* dst, int64_t capacity, rlt_snapshot_info* info,
                 hipStream_t stream);

/* Make the state equal to the snapshot: its positions, rings, memory, encoder cache and
 * pending encoder outputs are replaced (positions beyond the snapshot are dropped). The state
 * must have the snapshot's batch and ring layout, the same encoder-cache choice and max_len >=
 * n_encoded. Errors: INVALID_ARG (other configuration, batch, ring layout or cache choice),
 * STALE_STATE (other parameter values: caches computed with other weights are not
 * current-policy values, [R] §6.4), CAPACITY. Clears the state's staleness. */
int rlt_restore(rlt_model* m, rlt_state* s, const rlt_snapshot_info* info, const void* src, hipStream_t stream);

/* Behaviour sampling with recorded log-probabilities ([R] §6.2, Figure 4): for each of
 * `rows` rows of logits (device fp32, row stride ld >= vocab elements) draw
 *   tokens[b] = argmax_j (logits[b, j] / temperature + G(b, j)),  G = -log(-log U),
 * a draw from mu = softmax(logits[b] / temperature) over the whole vocabulary (Gumbel-max),
 * and write logprob[b] = log mu(tokens[b]) (nullable), the denominator of the importance
 * ratio. U(b, j) is a pure function of (seed, step, b, j): Philox4x64-10 (Salmon et al.,
 * SC 2011) with key (seed, 0), counter (j / 4, b, step, 0), output word j % 4, and
 * U = ((x >> 11) + 0.5) * 2^-53. Scores and the log-sum-exp are evaluated in float64.
 * temperature 0 is greedy decoding (lowest index on ties; logprob 0, a point mass). No
 * truncated sampling (top-k / top-p) is offered: [R] §6.2 notes that it breaks the support
 * condition p_Theta << mu of exact importance sampling.
 * tokens: device int32 [rows]. workspace (nullable): device memory of at least
 * rlt_sample_workspace bytes, 16-byte aligned; with it the 4096-id chunks of every row are
 * evaluated by separate workgroups side by side (the results are the same bit for bit).
 * Errors: INVALID_ARG (null, rows < 0, vocab < 1, ld < vocab, temperature negative or not
 * finite, workspace too small or misaligned), UNSUPPORTED (vocab > 2^20). Token ids are in
 * [0, vocab). */
int rlt_sample_workspace(int rows, int vocab, int64_t* bytes);
int rlt_sample(const float* logits, int rows, int vocab, int64_t ld, float temperature, uint64_t seed,
               uint64_t step, int32_t* tokens, float* logprob, void* workspace, int64_t workspace_bytes,
               hipStream_t stream);

/* rlt_sample for callers that cannot allocate (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the same draws and log mu, bit for bit, as
 * rlt_sample with a workspace, with the chunk statistics in a static device array of 1 MiB
 * that the library holds on every GPU it runs on until the process ends (its address is
 * looked up once per device, on the first call there). Calls no allocation routine. Every
 * call on a GPU uses that GPU's one array: calls that overlap on one GPU (different streams,
 * or different threads) race and give undefined results; calls ordered on one stream do not.
 * Capacity: rows * ceil(vocab / 4096) * 32 bytes <= 1 MiB (e.g. 4096 rows of a 32000-id
 * vocabulary); larger calls fail with CAPACITY before any launch. Other errors as rlt_sample. */
int rlt_sample_noalloc(const float* logits, int rows, int vocab, int64_t ld, float temperature, uint64_t seed,
                       uint64_t step, int32_t* tokens, float* logprob, hipStream_t stream);

/* Generation F.2 with on-device behaviour sampling ([S] appendix F.2; [R] §6.2 Figure 4):
 * consume `first` (device int32 [B], the last emitted token of every row: it is consumed
 * once before continuing), then n times: draw x_i ~ mu from the new logits as rlt_sample
 * does with draw index step0 + i, record tokens[b, i] = x_i and logprob[b, i] = log mu(x_i),
 * and consume x_i before the next draw, except the last one: tokens[:, n-1] is returned
 * unconsumed and is the next call's `first`. No host synchronisation between steps.
 * tokens int32 [B, n], logprob fp32 [B, n], logits fp32 [B, n, V] (nullable) on the device.
 * Needs keep_encoder_cache unless the state is at position 0. Errors: CAPACITY
 * (n_enc + n > max_len), ORDER (encoded positions not yet consumed), UNSUPPORTED,
 * STALE_STATE, INVALID_ARG. */
int rlt_generate(rlt_model* m, rlt_state* s, const int32_t* first, int n, float temperature, uint64_t seed,
                 uint64_t step0, int32_t* tokens, float* logprob, float* logits, hipStream_t stream);

/* Importance ratio of the replay contract ([R] §6.2 eq 5.5):
 * ratio[i] = exp(logprob_current[i] - logprob_behaviour[i]) for i < n, with the current
 * policy's log-probabilities from rlt_replay and the behaviour log-probabilities recorded
 * at sampling time. Device fp32 arrays; float64 inside. Errors: INVALID_ARG. */
int rlt_importance_ratio(const float* logprob_current, const float* logprob_behaviour, int64_t n, float* ratio,
                         hipStream_t stream);

/* Rows at their own positions (continuous batching; [S] appendix F.2 generation and [S]
 * appendix I.3 on RLT-2 generation with partial chunks, batched over rows that are at
 * unequal positions). rlt_step_rows consumes tokens[b] (device int32 [B]) for every row with
 * active[b] != 0 (HOST int32 [B]): encoder step, memory append and one transition at that
 * row's own position n_b + 1, logits of the moving rows in logits[b] (device fp32 [B, V];
 * rows that do not move get unspecified values there). Rows that do not move keep their
 * state exactly (their token is not read). RLT-2 rows update their register when their own
 * position closes a chunk. rlt_state_reset_rows returns the rows with rows[b] != 0 (host) to
 * H_0 (position 0, s = rho = s*), the others untouched: a finished sequence's row takes a new
 * sequence while the rest continue. Results per row equal an unbatched run of that row.
 * The first per-row call needs the state's encoded positions consumed (ORDER otherwise);
 * afterwards the batch-wide calls (encode, decode scan, step, generate, snapshot) accept the
 * state only while every row is at the same position (ORDER otherwise); reset and restore
 * return it to the batch-wide form. Per-row steps need keep_encoder_cache (UNSUPPORTED).
 * Errors: CAPACITY (a moving row at max_len), STALE_STATE, INVALID_ARG. */
int rlt_step_rows(rlt_model* m, rlt_state* s, const int32_t* tokens, const int32_t* active, float* logits,
                  hipStream_t stream);
int rlt_state_reset_rows(rlt_model* m, rlt_state* s, const int32_t* rows, hipStream_t stream);
/* Positions consumed by each row (host int32 [B]). */
int rlt_state_row_positions(const rlt_state* s, int32_t* n);

/* Full back-propagation through time of the replay ([R] §6.2 eq 5.5 for what is replayed;
 * [R] appendix B eq B.4 and §6.4: the reference training computation differentiates the
 * whole sequential unroll, through s_t, through every decoder key/value including entries
 * the window later drops, and through the encoder memory). For the loss
 *   L = sum_{b, t} dlogprob[b, t] * logprob[b, t]      (t = 1..T-1)
 * writes logprob (fp32 [B, T-1], as rlt_replay computes it) and dL/dtheta for every
 * manifest parameter. Any loss built from the replay's log-probabilities (an
 * importance-weighted policy objective, a likelihood) enters through its derivative with
 * respect to them, dlogprob (fp32 [B, T-1]).
 * Arithmetic is fp32 throughout (the log-sum-exp of the readout in float64) whatever
 * cfg->dtype: the weights are used as given. The unroll's intermediates live in `workspace`
 * (device memory the caller owns, at least rlt_replay_grad_workspace bytes for the same
 * checkpoint flag, 256-byte aligned); nothing is allocated. checkpoint = 0 keeps every
 * intermediate; checkpoint != 0 (activation checkpointing) keeps each block's input, the
 * decoder keys/values and the memory, and recomputes a position's block intermediates (an
 * encoder layer's, token-parallel) just before its backward: about a quarter of the
 * workspace for one more forward pass; weight gradients then accumulate position by position.
 * weights: the manifest tensors (device fp32, as for rlt_create, 16-byte aligned). grads: one writable
 * device fp32 tensor per manifest name with the same size (zeroed, then filled).
 * tokens: device int32 [B, T], x_1 = BOS. Asynchronous on `stream`.
 * Errors: INVALID_ARG (configuration, missing/unknown/duplicate/mis-sized tensors, B < 1,
 * T < 2, null pointers, workspace too small or misaligned), UNSUPPORTED (configuration
 * outside the library's limits). */
typedef struct {
  const char* name;
  float* data;
  int64_t numel;
} rlt_grad_tensor;

int rlt_replay_grad_workspace(const rlt_config* cfg, int B, int T, int checkpoint, int64_t* bytes);

int rlt_replay_grad(const rlt_config* cfg, const rlt_tensor* weights, int n_weights, rlt_grad_tensor* grads,
                    int n_grads, const int32_t* tokens, int B, int T, const float* dlogprob, float* logprob,
                    int checkpoint, void* workspace, int64_t workspace_bytes, hipStream_t stream);

/* Measurement aid: set the decoder of a state to have consumed its first n encoded
 * positions without running their transitions. s and the RLT-2 register keep their values
 * and every window ring slot is cleared to zero keys and values, so the next transition at
 * position n + 1 attends to zero-valued window entries at positions max(1, n-W+2)..n and
 * to the real memory prefix 1..n+1. The cost of a transition grows with its position
 * through the memory reads ([R] §4.2 eq 3.1 and 3.3: the per-step cost of the decoder
 * depends on t); this call lets a transition at a late position be timed, and checked, without
 * first running every earlier one. The resulting state is not the H_n of the method for
 * the encoded tokens. Requires n_decoded <= n <= n_encoded (RLT_ERR_ORDER otherwise). */
int rlt_state_seek(rlt_model* m, rlt_state* s, int n, hipStream_t stream);

/* Kernel timers (measurement). Kinds of launches that can be timed. */
typedef enum {
  RLT_TIME_MEMORY_ATTN = 0,    /* decoder cross-attention over the memory prefix ([S] §2.2) */
  RLT_TIME_WINDOW_ATTN = 1,    /* decoder sliding-window attention over the ring ([R] §3.3) */
  RLT_TIME_ENCODER_ATTN = 2,   /* encoder self-attention (prefill or over the encoder cache) */
  RLT_TIME_ENCODER_GEMM = 3,   /* encoder and memory-projection GEMMs (prefill, [S] §2.2) */
  RLT_TIME_DECODER_GEMM = 4,   /* merge, decoder block and readout GEMMs of the transitions */
  RLT_TIME_KINDS = 5
} rlt_time_kind;
/* With on != 0, every later launch of those kinds from the scan's launch path and the encoder
 * is bracketed by a pair of HIP events recorded on its stream (no device memory is allocated;
 * launches under stream capture are not timed). The timed launches of a per-row call cover
 * the launches of that call. Errors: INVALID_ARG. */
int rlt_kernel_timing(rlt_model* m, int on);
/* Sum of the event-timed durations (ms) and number of launches of one kind since the last
 * read; waits for the last recorded event, then clears the record. Errors: INVALID_ARG, HIP. */
int rlt_kernel_time(rlt_model* m, int kind, double* total_ms, int64_t* launches);

/* Scan driver for the decoder transitions: 0 = automatic (mode 1),
 * 1 = one launch sequence per position (stream-ordered), 2 = persistent cooperative kernel
 * with the automatic work split, 3 = persistent with every workgroup on all sequences,
 * 4/5/6 = persistent with 1/2/4 workgroups per CU, the workgroups of each XCD and dispatch
 * round forming an independent group that owns batch/8, batch/16 or batch/32 sequences
 * (falling back to fewer groups when the batch does not divide), 7/8 = mode 1 on 2/4 batch
 * slices each on its own stream, 9 = mode 1 with one position's launch sequence captured
 * once per state as a HIP graph and replayed (RLT-1; positions read from device memory).
 * The persistent kernel covers bf16 with d_head 64 or 128 only; other configurations use
 * mode 1 there. */
int rlt_set_scan_mode(rlt_model* m, int mode);

/* Batch-invariant arithmetic (on != 0): every kernel computes a row's result with the same
 * operations in the same order whatever the batch, the number of positions per call and the
 * serving split: the encoder runs its token-parallel positions through the decode GEMM and
 * the per-query attention kernel, the decoder normalises with the norm kernel instead of
 * the folded norms, and the scan uses the per-position launch path. Then a replay reproduces
 * the prefill + step (or rlt_generate) chain bit for bit, and at temperature 1 the importance
 * ratio of the replay against the recorded behaviour log-probabilities is exactly 1 ([R]
 * §6.3; the core.today essay on the method, §4-1, on sampler / trainer probabilities that
 * differ under one checkpoint until the kernels are batch-invariant: equal forward
 * probabilities need equal kernels, not only an equal schedule). Slower prefill; off by
 * default. */
int rlt_set_batch_invariant(rlt_model* m, int on);

/* Number of dependent decoder block passes issued since the state was reset
 * (T*L_D for RLT-1, ceil(T/K_c)*L_D for RLT-2 chunks, L_D per parallel RLT-0 pass;
 * [S] §2.7, Table 1). */
int rlt_state_block_steps(const rlt_state* s, int64_t* out);

/* Text of a status code. The codes name the conditions the pages' procedures rule out:
 * consuming positions the encoder has not produced ([S] appendix F.2: the last emitted token
 * is consumed before generation continues; RLT_ERR_ORDER), caches under other parameters
 * ([R] §6.4; RLT_ERR_STALE_STATE), and forms the pages do not define ([S] §2.2: G is 1 or L_D;
 * RLT_ERR_UNSUPPORTED). Returns a static string; never null. */
const char* rlt_status_string(int status);
/* Message of the calling thread's last failure (empty after none). Static storage per thread;
 * valid until that thread's next failing call. */
const char* rlt_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* RLT_H */
