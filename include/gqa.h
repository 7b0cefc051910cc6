/*
 * gqa.h - C ABI of the MI355X (gfx950) dense Qwen3-style GQA decoder library (libgqa355.so).
 *
 * The library evaluates the forward pass of a dense grouped-query-attention decoder: prefill
 * and incremental decode producing full-vocabulary FP32 logits, over a paged BF16 KV cache.
 * Every step runs in hand-written HIP kernels; there is no CPU fallback. Sources, by page and
 * section:
 *   Kipp Model Support, "The registry": dense Qwen3 decoders, BF16 weights, 8 KV heads of width
 *     128, vocabulary 151,936, RMS epsilon 1e-6, per-model RoPE theta and embedding tying.
 *   Kipp Model Support, "Validated results" (qwen3-0.6b-base): BF16 K/V storage contract;
 *     (qwen3-8b-base): untied lm_head.
 *   Kipp Model Support, "Quantization (Q8_0)": Q8_0 weights for the seven per-layer projections.
 *   Kipp Roadmap, status v0.0.2: per-session 32-position block table (bitwise equal to the
 *     contiguous layout), batched evaluation equal to isolated evaluation.
 *   Kipp Roadmap, status v0.0.3: model-owned KV slab shared by pooled sessions.
 *   Kipp Roadmap, status v0.0.4: device-derived prefill rounds; activation scratch per model.
 *   Kipp Reproducing, "Build": backend failures are fatal, never a silent fallback.
 *
 * Conventions
 *   - Every function returning int returns GQA_OK (0) or a negative GQA_E_* code; the message
 *     of the last failure on the calling thread is available from gqa_last_error(). A failing
 *     call leaves the model and session state unchanged, unless stated otherwise.
 *   - "device pointer" means memory of the model's HIP device (hipMalloc, or a torch CUDA
 *     tensor's data_ptr()); "host pointer" means ordinary CPU memory. The caller owns every
 *     buffer it passes; the library keeps no reference after the call returns (work it
 *     enqueued still reads/writes them in stream order).
 *   - `stream` is a hipStream_t of the model's device (NULL = the legacy default stream). All
 *     work is enqueued on it and the call returns without synchronising, except where stated.
 *     Calls on sessions of one model must be serialised on one stream: the activation scratch
 *     and the split-K partial buffers belong to the model.
 *   - Weights use row-major [out][in] matrices in the generator's logical layout (below).
 */
#ifndef GQA_H
#define GQA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GQA_OK 0
#define GQA_E_INVALID (-1)   /* bad argument or descriptor */
#define GQA_E_OOM (-2)       /* device memory or KV block pool exhausted */
#define GQA_E_DEVICE (-3)    /* no gfx950 device, or the current device is not gfx950 */
#define GQA_E_HIP (-4)       /* a HIP runtime call or kernel launch failed */
#define GQA_E_RANGE (-5)     /* token id outside [0, vocab) or context overflow */

#define GQA_SCHEME_BF16 0
#define GQA_SCHEME_Q8_0 1
#define GQA_SCHEME_AFFINE4 2   /* AFFINE4_GS32 (Kipp Model Support, "Quantization (AFFINE4_GS32)") */

#define GQA_MAX_BATCH 32
#define GQA_BLOCK_POSITIONS 32

typedef struct gqa_model gqa_model;
typedef struct gqa_session gqa_session;

/* Model shape (Kipp Model Support, "The registry"). n_kv_heads must be 8 and head_dim 128;
 * n_q_heads must be 16 or 32; hidden, 2*ffn and n_q_heads*128 must be multiples of 256 and
 * hidden <= 4096; vocab must be a multiple of 16. */
typedef struct {
  int32_t n_layers;
  int32_t hidden;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t ffn;
  int32_t vocab;
  int32_t tied;             /* 1: lm_head is the token embedding; 0: a separate lm_head */
  float rope_theta;
  float rms_eps;
  int32_t scheme;           /* GQA_SCHEME_BF16, _Q8_0 or _AFFINE4 (the seven projections) */
  int32_t kv_pool_blocks;   /* physical 32-position KV blocks in the model-owned pool */
  int32_t max_positions;    /* longest sequence any session may reach (RoPE table size) */
  int32_t max_round_tokens; /* prefill round width; 0 derives it from the device (CUs x 8) */
  int32_t prefill_operands; /* GQA_PREFILL_SPLIT (0): FP32 activations enter the prefill matrix-core
                               products as FP16 hi + lo (near-FP32); GQA_PREFILL_FP16 (1): as one
                               FP16 value (half the matrix-core work, FP16-rounded activations) */
  int32_t prefill_q8_direct; /* Q8_0 models: 0 (default): prefill GEMMs read FP16 copies of the
                               dequantised weights made at creation (one FP16 rounding of
                               scale * q; the BF16 GEMM speed); 1: they read the int8 quants and
                               scales directly (exact dequantisation, no copies, slower) */
  int32_t kv_quant;         /* KV cache format (Kipp Roadmap, status v0.0.4: the opt-in Q8_0 KV
                               cache, about 1.9x smaller than BF16). GQA_KV_BF16 (0): K/V stored
                               as BF16. GQA_KV_Q8_0 (1): each head row of 128 K or V values stored
                               as four Q8_0 blocks of 32 (int8 codes, fp16 scale = fp16(max|x|/127),
                               codes round(x / (max|x|/127)) half away from zero, the Q8_0 weight
                               rule): 136 bytes instead of 256. Attention reads
                               bf16(scale * code): the decode and prefill attention kernels widen
                               the codes as they load them; no BF16 copy is kept */
} gqa_model_desc;

#define GQA_PREFILL_SPLIT 0
#define GQA_PREFILL_FP16 1
#define GQA_KV_BF16 0
#define GQA_KV_Q8_0 1

/* Read-only facts about a created model. */
typedef struct {
  int32_t round_tokens;       /* prefill round width in use */
  int32_t cu_count;           /* compute units of the device */
  int64_t weight_bytes;       /* device bytes of all weights (Q8_0: quants + scales) */
  int64_t kv_pool_bytes;      /* device bytes of the K and V pools (with a Q8_0 cache: codes and
                                 scales) */
  int64_t scratch_bytes;      /* device bytes of per-model activation scratch */
  int64_t prefill_copy_bytes; /* device bytes of the FP16 copies prefill GEMMs read: projections
                                 (BF16, or dequantised Q8_0 / AFFINE4) and the padded lm_head */
  int32_t free_blocks;        /* KV blocks a new session can take: free, or cached and mapped by no session */
  int32_t cached_blocks;      /* KV blocks in the prefix cache (mapped or not) */
  int64_t prefix_lookups;     /* prefix-cache block lookups so far (pooled prefills) */
  int64_t prefix_hits;        /* lookups that mapped a cached block */
  int64_t prefix_evictions;   /* cached blocks evicted to make room */
} gqa_model_info;

/* Create a model on the current HIP device with seeded synthetic weights (Kipp Model Support,
 * "The registry": the dense Qwen3 decoders; the pages load checkpoints, this library generates
 * random-init weights of the same shape).
 * Weights: the counter-based generator documented in the library source (SplitMix64 outputs
 * summed Irwin-Hall style, scaled to std 0.02, rounded to BF16), one key per tensor derived
 * from `seed`; norm weights are 1.0. For GQA_SCHEME_Q8_0 the seven projections are then
 * quantised to Q8_0 (32-weight blocks, fp16 scale = max|w|/127, int8 quants); for
 * GQA_SCHEME_AFFINE4 to AFFINE4_GS32: per 32-weight group along a row an fp16 scale
 * fp16((max - min) / 15), an fp16 bias fp16(min) and 4-bit codes
 * q = clamp(round_half_away((w - bias) / scale), 0, 15) (FP32, from the stored scale and bias;
 * q = 0 when the scale is 0), w = scale * q + bias. Decode computes with these values exactly
 * (scale * sum(q x) + bias * sum(x) per group); prefill GEMMs read an FP16 rounding of them,
 * as they do for Q8_0 unless prefill_q8_direct is set.
 * Allocates weights, the KV pool and per-model scratch; fails with GQA_E_OOM if they do not
 * fit, GQA_E_DEVICE if the device is not gfx950, GQA_E_INVALID for a bad descriptor.
 * Synchronises the device before returning. *out is set only on success. */
int gqa_model_create(const gqa_model_desc* desc, uint64_t seed, gqa_model** out);

/* Free a model. All its sessions must have been destroyed. NULL is ignored. */
void gqa_model_destroy(gqa_model* model);

int gqa_model_get_info(const gqa_model* model, gqa_model_info* info);

/* Create a session that can hold `max_positions` positions. It takes
 * ceil(max_positions/32) physical blocks from the model pool:
 *   block_ids == NULL: the lowest-numbered free blocks, in increasing order (identity-like),
 *   then, if too few are free, cached prefix blocks no session maps, least recently used first;
 *   otherwise a host array of that many distinct, currently free block ids (any order:
 *   logical block i of the session lives in physical block block_ids[i]).
 * Returns GQA_E_OOM if the pool has too few free blocks, GQA_E_INVALID for a bad id list.
 * Uploads the block table (synchronously). */
int gqa_session_create(gqa_model* model, int32_t max_positions, const int32_t* block_ids, gqa_session** out);

/* Create a pooled session that can hold `max_positions` positions (Kipp Roadmap, status
 * v0.0.3: pooled sessions sharing one model-owned slab through a content-addressed pool of
 * 32-token blocks). It takes no blocks up front: a block is mapped when a position in it is
 * first written (GQA_E_OOM from that evaluation if no block is free or evictable).
 *   - Prefix reuse: gqa_session_eval_prefill with host ids at position 0 first maps the cached
 *     blocks holding the prompt's leading whole 32-token blocks (matched by token ids and by the
 *     chain of blocks before them, compared exactly, not by hash alone), keeping at least one id
 *     to evaluate, and evaluates only the rest; gqa_session_reused reports how many positions
 *     it took. Its logits equal those of evaluating the whole prompt, up to rounding.
 *   - Publishing: gqa_session_destroy and gqa_session_reset (the end of a request) publish the
 *     session's whole blocks whose ids it knows (those evaluated from host ids), from the first
 *     block on, into the cache; gqa_session_publish does so without ending the request.
 *   - Cached blocks stay in the model's pool after their sessions end; when a block is needed
 *     and none is free, the least recently used cached block that no session maps is evicted.
 *   - Writing into a cached block (after gqa_session_truncate) first gives the session a
 *     private copy of it, so other sessions' blocks never change.
 * Blocks are handed from one session to another on the host as soon as a call returns, so all
 * sessions of a model must enqueue their work on one stream (as the model's scratch already
 * requires). The device table is updated on the evaluation's stream. */
int gqa_session_create_pooled(gqa_model* model, int32_t max_positions, gqa_session** out);

/* Publish a pooled session's whole known blocks below its position now (see
 * gqa_session_create_pooled). GQA_E_INVALID for a session with a fixed table. */
int gqa_session_publish(gqa_session* session);

/* Positions the session's last gqa_session_eval_prefill took from the prefix cache (0 for
 * sessions with a fixed table). */
int32_t gqa_session_reused(const gqa_session* session);

/* Return the session's blocks to the pool and free it (a pooled session publishes first).
 * NULL is ignored. */
void gqa_session_destroy(gqa_session* session);

/* Set the position to 0. A session with a fixed table keeps its blocks; a pooled session
 * publishes and then gives up its blocks. */
int gqa_session_reset(gqa_session* session);

/* Number of positions evaluated so far. */
int32_t gqa_session_position(const gqa_session* session);

/* Append n >= 1 prompt tokens (host array of ids in [0, vocab)) at positions
 * [pos, pos + n), in rounds of the model's round width, and write the logits of the last new
 * position to `logits` (device, vocab floats) and its argmax (lowest index on ties) to
 * `argmax` (device, one int32; may be NULL). GQA_E_RANGE if an id is out of range or
 * pos + n exceeds the session's max_positions. */
int gqa_session_eval_prefill(gqa_session* session, const int32_t* ids, int32_t n, float* logits, int32_t* argmax,
                             hipStream_t stream);

/* As gqa_session_eval_prefill with the n ids already in device memory (`ids`, read on
 * `stream`; the caller keeps them alive until the call's work completes), so no host copy is
 * made. Ids cannot be checked synchronously: an id outside [0, vocab) makes its embedding row
 * NaN (hence the logits NaN and the argmax -1) and sets the model's sticky device error (see
 * gqa_model_check_device_error); the position still advances. GQA_E_RANGE for a context
 * overflow. (Kipp Roadmap, status v0.0.4: prompt rounds evaluated on the device.) */
int gqa_session_eval_prefill_device(gqa_session* session, const int32_t* ids, int32_t n, float* logits,
                                    int32_t* argmax, hipStream_t stream);

/* Multi-row evaluation (Kipp Roadmap, status v0.0.2: logits for several positions from one
 * call). Appends n >= 1 host ids like gqa_session_eval_prefill, but writes the logits of every
 * new position: logits [n][vocab] (device, row i is position pos + i) and, when `argmax` is
 * not NULL, argmax [n] (device, lowest index on ties). Row n-1 equals what eval_prefill
 * writes for the same call. Errors as eval_prefill. */
int gqa_session_eval_n(gqa_session* session, const int32_t* ids, int32_t n, float* logits, int32_t* argmax,
                       hipStream_t stream);

/* Multi-row scoring (Kipp Roadmap, status v0.0.3: tolerance-bound scoring of several rows).
 * Appends n >= 2 host ids like gqa_session_eval_prefill and writes scores [n-1] (device):
 * scores[i] = log softmax(logits of position pos + i)[ids[i + 1]], the natural-log
 * probability of each id given the ones before it (the sum of -scores is the negative
 * log-likelihood a perplexity is built from). No logits are returned. The log-softmax is taken
 * in FP32 over the FP32 logits. GQA_E_INVALID for n < 2; otherwise errors as eval_prefill. */
int gqa_session_eval_scored(gqa_session* session, const int32_t* ids, int32_t n, float* scores, hipStream_t stream);

/* Truncate the session to its first `pos` positions (0 <= pos <= current position), so the
 * next evaluation continues at `pos`; the KV of later positions is overwritten as they are
 * evaluated again. Resuming after a truncation gives the same logits as evaluating the kept
 * prefix and the new tokens from scratch (Kipp Model Support, "What the gates check":
 * truncate/resume among the compared paths). GQA_E_RANGE for pos out of range. Host-only,
 * no device work: call it once the previous evaluation's stream work is ordered before the
 * next. */
int gqa_session_truncate(gqa_session* session, int32_t pos);

/* Evaluate one token at the session's position: incremental decode over the session's KV cache
 * (Kipp Model Support, "What the gates check": cached decode equal to recomputation without the
 * cache, at every decode position). `id` is a host pointer when id_on_device is
 * 0 (validated: GQA_E_RANGE if outside [0, vocab)) or a device pointer when 1 (for greedy
 * loops without host round trips, e.g. the previous call's argmax buffer). A device id
 * outside [0, vocab) cannot be reported synchronously: its logits become NaN, argmax -1, and
 * the model's sticky device error is set (see gqa_model_check_device_error); the position
 * still advances. Writes vocab logits and the argmax like eval_prefill. */
int gqa_session_eval_decode(gqa_session* session, const int32_t* id, int32_t id_on_device, float* logits,
                            int32_t* argmax, hipStream_t stream);

/* One token for each of B distinct sessions of the same model (1 <= B <= 32; Kipp Roadmap, status
 * v0.0.2: batched evaluation, gated equal to isolated evaluation): row b of
 * `ids` (host or device per ids_on_device, as for eval_decode) is evaluated at sessions[b]'s
 * position. Writes logits [B][vocab] and argmax [B] (device). Row b is bit-identical to
 * gqa_session_eval_decode on sessions[b] alone. GQA_E_INVALID for duplicate sessions, mixed
 * models or B out of range; GQA_E_RANGE for context overflow or a host id out of range. */
int gqa_session_eval_batch(gqa_session* const* sessions, int32_t B, const int32_t* ids, int32_t ids_on_device,
                           float* logits, int32_t* argmax, hipStream_t stream);

/* Allocation-free single-row decode, for callers that cannot allocate device memory during a
 * call: code recorded under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation. Same arguments, arithmetic, kernels and results (bit for bit) as
 * gqa_session_eval_decode, but the call's scratch -- residual stream, projection outputs,
 * operand rows, attention chunk partials and arrival counters, sums of squares, argmax
 * candidates -- lives in a static device array of the library (2 MiB per device, held by each
 * device the library runs on until the process ends) instead of the model's buffers. The call
 * allocates and frees nothing. Limits: the model's decode must fit the whole-K matvec path
 * (hidden, attention width and ffn <= 16380) and its row scratch must fit 2 MiB (the Qwen3-8B
 * shape needs about 1.3 MiB; the size grows with vocab / 2 bytes and n_q_heads x 33 KiB);
 * otherwise GQA_E_INVALID with the needed size, before any work is enqueued. BF16 and Q8_0 KV
 * caches are both supported. The current device must be the model's (GQA_E_INVALID otherwise). Every call on a
 * device shares that device's array, which keeps the last call's contents (the arrival
 * counters that must start at zero are cleared by the call itself): calls that overlap on one
 * device -- on different streams, or from different models -- race and must not be made. */
int gqa_session_eval_decode_static(gqa_session* session, const int32_t* id, int32_t id_on_device, float* logits,
                                   int32_t* argmax, hipStream_t stream);

/* Synchronise `stream`, then return GQA_E_RANGE (and clear the flag) if a device-resident
 * token id was out of range since the last check; GQA_E_HIP (and clear it) if a decode
 * launch gave up waiting for the launch before it (the decode of at most four rows orders its
 * per-layer launches through device counters with a bounded wait; the results of that call
 * are invalid); else GQA_OK. */
int gqa_model_check_device_error(gqa_model* model, hipStream_t stream);

/* Kernel timing with HIP events on the caller's stream, for roofline reports: while a class is
 * selected, every launch of that kernel class is bracketed by a pair of events.
 * gqa_model_profile(model, cls) starts a new recording (cls = GQA_PROF_NONE stops);
 * gqa_model_profile_read synchronises the device and returns the launch count and the summed
 * event time in milliseconds of the current recording. At most 65,536 launches are recorded;
 * later ones are counted in *dropped. While GQA_PROF_DECODE_GATEUP is selected, decode calls
 * issue their per-layer launches as ordinary dependent launches (not the any-order chain they
 * use otherwise, whose launches start early and wait), so each event pair brackets the
 * kernel's own execution; the results are the same bits. */
#define GQA_PROF_NONE 0
#define GQA_PROF_DECODE_GATEUP 1   /* decode gate/up matvec with SwiGLU (HBM bound) */
#define GQA_PROF_PREFILL_GATEUP 2  /* prefill gate/up GEMM with SwiGLU (matrix-core bound) */
#define GQA_PROF_PREFILL_ATTN 3    /* prefill flash attention */
#define GQA_PROF_DECODE_LMHEAD 4   /* decode lm_head matvec */
#define GQA_PROF_ROWS_LMHEAD 5     /* lm_head over a group of up to 32 rows in eval_n / eval_scored */
int gqa_model_profile(gqa_model* model, int32_t kernel_class);
int gqa_model_profile_read(gqa_model* model, int64_t* launches, double* total_ms, int64_t* dropped);

/* Test hook of the bounded wait in the decode chain (see gqa_model_check_device_error), not for
 * production use. While `offset` > 0 every chained decode launch of this model waits for `offset`
 * more arrivals per counter than any launch makes: the first waiting launch gives up after its
 * bounded wait (about 2^16 polls) and sets the model's error word, the later ones give up at
 * once, and the call completes with invalid results (the session's KV rows written by it are
 * invalid too) while gqa_model_check_device_error reports GQA_E_HIP. 0 (the default) restores
 * normal operation. GQA_E_INVALID for an offset outside [0, 2^20]. */
int gqa_model_debug_chain_offset(gqa_model* model, int32_t offset);

/* Message of the last failure on this thread ("" if none). Valid until the next call. */
const char* gqa_last_error(void);

/* Build record baked into the library when it was compiled (Kipp Reproducing, "Benchmarks":
 * every benchmark record carries the commit, whether the tree was dirty, the binary and the
 * compiler): a static JSON object string with "commit" (git HEAD at build time, or null),
 * "dirty" (true / false, or null when unknown), "sources_sha256" (hash of the library's
 * sources and header), "hipcc" (the compiler's version line), "flags" and "built_utc". Never
 * NULL; owned by the library. */
const char* gqa_build_info(void);

/* Hardware record of HIP device `device` for benchmark records (same source): fills *out.
 * GQA_E_INVALID for a device index out of range or a NULL out; GQA_E_HIP if the runtime
 * query fails. Does not require a gfx950 device (it only reports). */
typedef struct {
  char name[256];           /* marketing name reported by the runtime */
  char arch[64];            /* gcnArchName, e.g. "gfx950:sramecc+:xnack-" */
  int32_t cu_count;         /* compute units */
  int32_t clock_khz;        /* peak shader clock reported by the runtime */
  int32_t memory_clock_khz; /* peak memory clock reported by the runtime */
  int32_t memory_bus_bits;  /* memory bus width */
  int64_t total_memory;     /* device memory bytes */
  int64_t l2_bytes;         /* L2 bytes as reported */
  int64_t lds_per_cu;       /* LDS bytes per compute unit */
  int32_t runtime_version;  /* hipRuntimeGetVersion */
  int32_t driver_version;   /* hipDriverGetVersion */
} gqa_device_desc;
int gqa_device_describe(int32_t device, gqa_device_desc* out);

/* ---- inspection, for tests (synchronous) ---- */

/* Tensor kinds for gqa_debug_read_weight, in the generator's order. */
#define GQA_T_EMBED 0
#define GQA_T_ATTN_NORM 1
#define GQA_T_Q 2
#define GQA_T_K 3
#define GQA_T_V 4
#define GQA_T_Q_NORM 5
#define GQA_T_K_NORM 6
#define GQA_T_O 7
#define GQA_T_FFN_NORM 8
#define GQA_T_GATE 9
#define GQA_T_UP 10
#define GQA_T_DOWN 11
#define GQA_T_FINAL_NORM 12
#define GQA_T_LM_HEAD 13

/* Copy `rows` logical rows starting at `row0` of a BF16 tensor (before any Q8_0
 * quantisation the library does not keep BF16 copies of Q8_0 projections: GQA_E_INVALID)
 * into `dst` (host, rows x cols uint16 BF16 bits, row-major in the logical [out][in] layout). */
int gqa_debug_read_weight(gqa_model* model, int32_t kind, int32_t layer, int32_t row0, int32_t rows, uint16_t* dst);

/* For a Q8_0 model: copy logical rows [row0, row0+rows) of a projection as int8 quants
 * (rows x cols) and fp16 scale bits (rows x cols/32) into host buffers. */
int gqa_debug_read_q8(gqa_model* model, int32_t kind, int32_t layer, int32_t row0, int32_t rows, int8_t* quants,
                      uint16_t* scales);

/* For an AFFINE4 model: copy logical rows [row0, row0+rows) of a projection as 4-bit codes (one
 * per byte, rows x cols), fp16 scale bits and fp16 bias bits (rows x cols/32 each) into host
 * buffers. */
int gqa_debug_read_affine4(gqa_model* model, int32_t kind, int32_t layer, int32_t row0, int32_t rows, uint8_t* codes,
                           uint16_t* scales, uint16_t* biases);

/* Copy the BF16 bits of K and V of `layer` for logical positions [pos0, pos0+n) of a session,
 * read through its block table, into host arrays of n x 8 x 128 uint16 each (with a Q8_0 cache:
 * the values attention reads, bf16(scale * code)). GQA_E_INVALID for a position whose block a
 * pooled session has not mapped. */
int gqa_debug_read_kv(gqa_session* session, int32_t layer, int32_t pos0, int32_t n, uint16_t* k, uint16_t* v);

/* For a model with a Q8_0 KV cache: copy the int8 codes (n x 8 x 128 each) and the fp16 scale bits
 * (n x 8 x 4 each) of K and V of `layer` for logical positions [pos0, pos0+n) of a session into
 * host arrays. GQA_E_INVALID if the cache is BF16 or a position is unmapped. */
int gqa_debug_read_kv_q8(gqa_session* session, int32_t layer, int32_t pos0, int32_t n, int8_t* kcodes,
                         uint16_t* kscales, int8_t* vcodes, uint16_t* vscales);

/* Activation scratch buffers of the model (contents are those left by the last call; layouts
 * are internal and may change): copy elements [offset, offset + count) of buffer `which` into
 * host memory `dst` (FP32 buffers 4 bytes per element, FP16 buffers 2). */
#define GQA_S_RESID_A 0   /* FP32 residual stream (prefill rows / decode rows) */
#define GQA_S_RESID_B 1   /* FP32 second residual buffer (split-K decode path) */
#define GQA_S_PART_A 2    /* FP32 projection outputs or split partials */
#define GQA_S_PART_B 3
#define GQA_S_ATTN_HI 4   /* FP16 hi / lo of the attention output (o projection operand) */
#define GQA_S_ATTN_LO 5
#define GQA_S_MLP_HI 6    /* FP16 hi / lo of silu(gate) * up (down projection operand) */
#define GQA_S_MLP_LO 7
#define GQA_S_NORM_HI 8   /* FP16 hi / lo of normalised rows (prefill projection operand, lm_head) */
#define GQA_S_NORM_LO 9
#define GQA_S_SUMSQ 10    /* FP32 per-range sums of squares [2][8][32] */
#define GQA_S_QROT 11     /* FP32 normed, rotated q of a prefill round */
#define GQA_S_QKV 12      /* FP32 q|k|v projection of a prefill round */
int gqa_debug_read_scratch(gqa_model* model, int32_t which, int64_t offset, int64_t count, void* dst);

/* Copy the FP32 RoPE tables (positions [0, n) x 64 cos, then sin) into host arrays. */
int gqa_debug_read_rope(gqa_model* model, int32_t n, float* cos_out, float* sin_out);

#ifdef __cplusplus
}
#endif
#endif /* GQA_H */
