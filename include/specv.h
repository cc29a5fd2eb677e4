/*
 * specv.h -- C ABI of libspecv, the gfx950 (MI355X) verify transaction of
 * greedy speculative decoding.
 *
 * The transaction (pegainfer page "DFlash speculative decoding", transaction
 * section; TensorSharp speculative decoding page, protocol section):
 *   propose K drafts -> ONE trunk forward over the span [last, d1..dK] that
 *   yields the trunk argmax a0..aK of every row -> accept_greedy keeps the
 *   longest prefix with d(i) == a(i-1) and adds the trunk's own token a(m),
 *   so 1..K+1 tokens are committed -> the KV rows of [last, d1..dm] are kept
 *   and the cache length becomes p+m+1 (draft-seed alignment paragraph of the
 *   pegainfer page); rejected rows stay past the length and are overwritten
 *   later (coreai-model-zoo dense n-gram note, KV-only rollback paragraph).
 *
 * General rules for every call:
 *   - Return value: 0 on success, a negative SPEC_E* code on failure; no call
 *     aborts or throws.  spec_last_error() gives the message of the last
 *     failure on that context (or of the last spec_create failure for NULL).
 *   - Device memory is owned by the caller (allocated with PyTorch): the
 *     weight arena, the KV pool and the workspace are passed to spec_create
 *     and must outlive the context.  The library never allocates device
 *     memory.  It owns only host state and HIP graph objects.
 *   - Host arrays passed to a call are borrowed for the duration of the call.
 *   - One context per HIP stream; a context is not thread-safe.  Every
 *     launch and copy is issued on the stream given to spec_create, and the
 *     transaction calls return only after their results reached the host.
 *   - Tokens are int32 in [0, vocab).
 */
#ifndef SPECV_H
#define SPECV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPEC_API __attribute__((visibility("default")))

/* ------------------------------------------------------------ error codes */
#define SPEC_OK 0
#define SPEC_EINVAL (-1)    /* bad argument: K out of range, token outside [0,vocab), NULL, bad id */
#define SPEC_ECAPACITY (-2) /* p+K+1 > max_ctx, no free KV block, buffer too small (admission refusal) */
#define SPEC_ESTATE (-3)    /* verify before prefill, rewind beyond the cache, weights not loaded */
#define SPEC_EHIP (-4)      /* a HIP runtime call failed; the message holds hipGetErrorString */
#define SPEC_ENAN (-5)      /* a logit row held NaN: the argmax is undefined */

/* --------------------------------------------------------- model and flags */
#define SPEC_WFMT_BF16 0     /* bf16 weights, canonical [out][in] row-major                   */
#define SPEC_WFMT_INT4G128 1 /* int4 group-128: q4 uint8 [out][in/2] (low nibble = even col)  */
                             /* plus bf16 scales [out][in/128]; w = scale * q, q in [-8, 7]    */

#define SPEC_FLAG_KEEP_LOGITS 1u /* also store every row's logits (fp32) for spec_debug_logits */
#define SPEC_FLAG_NO_GRAPH 2u    /* launch each kernel eagerly instead of replaying a HIP graph */

#define SPEC_MAX_SPAN 16    /* rows per sequence per forward (K <= 15)      */
#define SPEC_MAX_ROWS 128   /* rows per forward over all sequences           */
#define SPEC_BLOCK_TOKENS 16 /* tokens per KV block                          */

typedef struct spec_model_desc {
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
  int32_t weight_format; /* SPEC_WFMT_*; the embedding is always bf16 */
  float rms_eps;         /* RMSNorm epsilon */
  double rope_theta;     /* RoPE base; rotate-half pairs (i, i + head_dim/2) */
  int32_t max_ctx;       /* tokens per sequence, including the verify span */
  int32_t max_seqs;      /* sequences the KV pool serves */
  int32_t max_rows;      /* rows per forward (n_seq * (K+1)), 1..SPEC_MAX_ROWS */
  int32_t n_blocks;      /* 16-token KV blocks in the pool (0: max_seqs*ceil(max_ctx/16)) */
  uint32_t flags;        /* SPEC_FLAG_* */
  /* Sliding-window layers (TensorSharp page, sliding-window section): each
   * layer l < 64 with bit l of swa_layers set attends, from a row at position
   * t, only the keys at positions [t - swa_window + 1, t], and keeps its KV
   * rows in a ring per sequence of swa_window + 16 slots (rounded up to whole
   * 16-token blocks).  A verify writes its rows at their true positions; the
   * ring's 16 spare slots are what keeps every position any row (of this
   * verify, or after a partial rejection) still attends to, so rewinding a
   * ring layer is exact and nothing is backed up.  0: no sliding window. */
  int32_t swa_window;
  int32_t reserved;      /* 0 */
  uint64_t swa_layers;
  /* Recurrent layers (TensorSharp page, recurrent-trunk section): each layer
   * l < 64 with bit l of rec_layers set is a delta-rule layer instead of
   * attention -- per kv head a state S [head_dim][head_dim] that every row
   * updates with its unit key k and value v, S <- S + rec_beta (v - S k) k^T,
   * and every query head of the group reads with its unit query, o = S q (no
   * rotary embedding).  A verify stores the state after every span row and
   * the accept stage commits the one after the last kept row on the device
   * (no copy, no second forward).  Such a model rewinds only to 0.  Not
   * combined with a sliding window on the same layer; at most 8 query heads
   * per kv head; rec_beta in (0, 1]. */
  uint64_t rec_layers;
  float rec_beta;
  int32_t reserved2;     /* 0 */
} spec_model_desc;

/* Sizes of the caller-owned buffers for a description. */
typedef struct spec_buffer_sizes {
  size_t weights_bytes;   /* device: packed weight arena */
  size_t kv_bytes;        /* device: fp16 KV block pool */
  size_t workspace_bytes; /* device: activations, partial sums, counters, tables */
  size_t host_bytes;      /* pinned host: staging of spans and results */
} spec_buffer_sizes;

typedef struct spec_device_buffers {
  void* weights;   size_t weights_bytes;
  void* kv;        size_t kv_bytes;
  void* workspace; size_t workspace_bytes;
  void* host;      size_t host_bytes; /* pinned (page-locked) host memory */
} spec_device_buffers;

typedef struct spec_ctx spec_ctx;

/* Matrix and norm identifiers for the weight loaders. */
#define SPEC_MAT_Q 0    /* [n_q*head_dim][hidden]  */
#define SPEC_MAT_K 1    /* [n_kv*head_dim][hidden] */
#define SPEC_MAT_V 2    /* [n_kv*head_dim][hidden] */
#define SPEC_MAT_O 3    /* [hidden][n_q*head_dim]  */
#define SPEC_MAT_GATE 4 /* [ffn][hidden]           */
#define SPEC_MAT_UP 5   /* [ffn][hidden]           */
#define SPEC_MAT_DOWN 6 /* [hidden][ffn]           */
#define SPEC_MAT_EMB 7  /* [vocab][hidden], bf16 in every format */
#define SPEC_MAT_LM 8   /* [vocab][hidden]         */
#define SPEC_NORM_ATTN 0
#define SPEC_NORM_FFN 1
#define SPEC_NORM_FINAL 2

/* Buffer sizes for `desc`: the caller allocates all four (the library never
 * allocates device memory).  Sizing everything up front is how an admission
 * that cannot fit is refused cleanly before any work starts (pegainfer page,
 * memory section: a request that does not fit is rejected at admission).
 * EINVAL for an unsupported description. */
SPEC_API int spec_query_buffers(const spec_model_desc* desc, spec_buffer_sizes* out);

/* Create a context over caller-owned buffers (each at least the size
 * spec_query_buffers gives, device pointers 256-byte aligned) on `hip_stream`
 * (a hipStream_t; not the legacy NULL stream, since forwards are captured into
 * HIP graphs).  Clears the KV pool and the workspace.  Weights are then loaded
 * with spec_load_matrix / spec_load_norm. */
SPEC_API int spec_create(const spec_model_desc* desc, const spec_device_buffers* bufs, void* hip_stream,
                spec_ctx** out);
/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * context with the library's own static scratch, SPEC_STATIC_SCRATCH_BYTES
 * per GPU (held until the process ends), as its workspace.  bufs carries the
 * weights, the KV pool and the pinned host staging as for spec_create; its
 * workspace must be NULL with size 0.  The context launches its kernels
 * eagerly (no HIP graph objects) and keeps no timing events, so no call on it
 * allocates device memory; spec_get_stats leaves forward_ms_by_span at zero.
 * One static context per GPU at a time: a second spec_create_static on the
 * same device fails with ESTATE until the first is destroyed (calls on two
 * would race on the one scratch).  ECAPACITY when the description needs more
 * workspace than the scratch holds (spec_query_buffers gives the need);
 * EHIP if the scratch's device address cannot be obtained. */
#define SPEC_STATIC_SCRATCH_BYTES (32u << 20)
SPEC_API int spec_create_static(const spec_model_desc* desc, const spec_device_buffers* bufs, void* hip_stream,
                                spec_ctx** out);
SPEC_API int spec_destroy(spec_ctx* ctx);
SPEC_API const char* spec_last_error(const spec_ctx* ctx);

/* Repack one canonical matrix from device memory into the arena.  `src` is
 * bf16 [rows][cols] (or, for int4 models and which != SPEC_MAT_EMB, q4 bytes
 * with `scales` bf16 [rows][cols/128]).  layer is ignored for EMB and LM.
 * Synchronous; `src` may be freed on return. */
SPEC_API int spec_load_matrix(spec_ctx* ctx, int layer, int which, const void* src, const void* scales);
/* Copy one fp32 gain vector [hidden] from device memory. */
SPEC_API int spec_load_norm(spec_ctx* ctx, int layer, int which, const float* src);

/* ---------------------------------------------------------- transaction */

/* Batch-1 calls act on sequence 0.
 * spec_prefill: empty the sequence, forward the prompt (rows 0..n-1, in
 * chunks of up to SPEC_MAX_SPAN rows, each committing all its rows) and
 * return g0 = argmax of the last prompt row.  g0 is not cached; it is span[0]
 * of the first verify, which writes its KV row (pegainfer page, draft-seed
 * alignment paragraph: the first verify after prefill starts from the token
 * prefill produced).  Prefill itself is the plain forward: speculation only
 * changes decoding (TensorSharp page, benchmarks paragraph).  On any failure
 * (ENAN, EHIP) the sequence is left empty on the host and the device. */
SPEC_API int spec_prefill(spec_ctx* ctx, const int32_t* tokens, int n, int32_t* next_token);

/* spec_verify: span = [last, d1..dK], K in [0, SPEC_MAX_SPAN-1]; span[0] is
 * the token for position p = cache length.  Writes argmax[0..K] (the trunk
 * argmax of every row, lowest index on ties) and *accept_len = m in [0, K];
 * the committed tokens are argmax[0..m] and the cache length becomes p+m+1
 * (set on the device by the accept kernel).  K = 0 is a plain decode step. */
SPEC_API int spec_verify(spec_ctx* ctx, const int32_t* span, int K, int32_t* argmax, int32_t* accept_len);

/* spec_rewind: shorten the cache to len (0 <= len <= cache length; a model
 * with recurrent layers only to 0 or its current length); rows past
 * len stay in memory and are overwritten by later forwards (TensorSharp page,
 * interfaces section: SpecRewindCache(length); coreai note, KV-only rollback
 * paragraph: rolling back is not advancing the position).  Used for budget or
 * stop truncation and by the verify-cost sweep.  ESTATE outside [0, length].
 * spec_cache_len: the current cache length (TensorSharp page, interfaces
 * section: CacheSeqLen). */
SPEC_API int spec_rewind(spec_ctx* ctx, int len);
SPEC_API int spec_cache_len(spec_ctx* ctx, int* len);

/* Multi-sequence calls over the paged pool (16-token blocks).
 * spec_verify_batch: n_seq distinct sequences (seq_ids), each with a span of
 * K+1 tokens, spans row-major [n_seq][K+1]; n_seq*(K+1) <= max_rows.  Writes
 * argmax [n_seq][K+1] and accept_len [n_seq]; each sequence advances by its
 * own m+1.  Blocks past a sequence's new length return to the free pool. */
SPEC_API int spec_prefill_seq(spec_ctx* ctx, int seq, const int32_t* tokens, int n, int32_t* next_token);
SPEC_API int spec_verify_batch(spec_ctx* ctx, int n_seq, const int32_t* seq_ids, const int32_t* spans, int K,
                      int32_t* argmax, int32_t* accept_len);
/* spec_verify_batch_k: the same step where each sequence b proposed its own
 * drafts[b] in [0, K] drafts (spans[b][1..drafts[b]]); the rest of its span
 * row, spans[b][drafts[b]+1..K], is padding (any valid token).  Every
 * sequence runs the full K+1 rows, so the step keeps one shape and one
 * captured graph whatever the mix (pegainfer page, CUDA-graph section: a
 * graph captured at a short span and replayed at a longer one under-computes
 * the tail; here padding plus a per-sequence draft count replaces shorter
 * spans).  The accept stage counts only a sequence's real drafts: m[b] <=
 * drafts[b], the cache advances by m[b]+1, and argmax rows past drafts[b] are
 * computed on padding and carry no meaning.  drafts == NULL is
 * spec_verify_batch (K drafts each).  EINVAL for a count outside [0, K]. */
SPEC_API int spec_verify_batch_k(spec_ctx* ctx, int n_seq, const int32_t* seq_ids, const int32_t* spans, int K,
                                 const int32_t* drafts, int32_t* argmax, int32_t* accept_len);
SPEC_API int spec_rewind_seq(spec_ctx* ctx, int seq, int len);
SPEC_API int spec_cache_len_seq(spec_ctx* ctx, int seq, int* len);
/* Free every block of a sequence (cache length 0). */
SPEC_API int spec_release_seq(spec_ctx* ctx, int seq);

/* Sampled verification (TensorSharp page, protocol section, the verify step:
 * the sampler draws a token from every row and drafts are accepted while the
 * drawn token matches; the first mismatching row's draw is the corrected
 * token).  temperature 0 (the default) is greedy: every row's token is its
 * argmax.  temperature > 0: row i of a span at position p + i draws
 * argmax_v (logit_v / temperature + g_v) -- a draw from softmax(logit /
 * temperature) -- with Gumbel noise g_v = -log(-log u_v) and u_v from
 * Philox4x32-10 keyed by `seed` at the counter (v / 4, p + i, sequence id, 0),
 * word v % 4.  A draw depends on (seed, sequence, position, v) only, so
 * speculation leaves the sampled stream exactly as plain sampled decoding
 * would draw it.  Applies to every later forward of the context (prefill's
 * g0 included), on the device inside the LM-head epilogue; argmax outputs
 * then hold the drawn tokens.  EINVAL for a negative or non-finite
 * temperature. */
SPEC_API int spec_set_sampling(spec_ctx* ctx, float temperature, uint64_t seed);

/* Logits of the rows of the last forward, fp32 [rows][vocab]; only for a
 * context created with SPEC_FLAG_KEEP_LOGITS.  rows <= rows of that forward.
 * For checking only: the per-row logits of the multi-row forward (TensorSharp
 * page, interfaces section, SpecForward with every row's logits), compared
 * row by row with a reference under teacher forcing (TensorSharp page, parity
 * section).  host_out: caller-owned [rows][vocab] floats.  ESTATE without the
 * flag, EINVAL for rows outside [0, rows of the last forward]. */
SPEC_API int spec_debug_logits(spec_ctx* ctx, float* host_out, int rows);

/* --------------------------------------------------------- measurement */

typedef struct spec_stats {
  int64_t forwards;               /* forwards launched (prefill chunks included) */
  int64_t verify_calls;           /* spec_verify + spec_verify_batch calls */
  int64_t drafted, accepted;      /* drafts submitted / accepted over verify calls */
  int64_t forwards_by_span[SPEC_MAX_SPAN + 1]; /* verify forwards by rows per sequence */
  int64_t graphs;                 /* HIP graphs instantiated */
  double forward_ms_by_span[SPEC_MAX_SPAN + 1]; /* summed device time of those forwards (HIP events
                                                  * on the context stream around each forward) */
} spec_stats;
SPEC_API int spec_get_stats(spec_ctx* ctx, spec_stats* out);

/* Time `iters` verify forwards of span length S (= K+1) over one sequence at
 * its current cache length, measured with HIP events on the context stream
 * from graph launch to the accept kernel's end, host excluded.  The cache is
 * left unchanged (the forwards run in a no-commit mode).  spans: [iters][S]
 * tokens; ms_out: [iters]. */
SPEC_API int spec_time_verify(spec_ctx* ctx, int S, int iters, const int32_t* spans, float* ms_out);

/* Per-kernel-class timing of `iters` eager forwards of span S at the current
 * cache length (no commit): HIP events bracket every launch on the context
 * stream.  us_out[SPEC_OP_COUNT] = mean microseconds per launch of each class,
 * launches_out[SPEC_OP_COUNT] = launches per forward. */
#define SPEC_OP_EMBED 0
#define SPEC_OP_QKV 1
#define SPEC_OP_ATTN 2
#define SPEC_OP_O 3
#define SPEC_OP_GATEUP 4
#define SPEC_OP_DOWN 5
#define SPEC_OP_LM 6
#define SPEC_OP_COUNT 7
SPEC_API int spec_profile_ops(spec_ctx* ctx, int S, int iters, const int32_t* spans, float* us_out,
                     int32_t* launches_out);

/* Mean microseconds per launch of one op class launched back to back: `reps`
 * passes over every layer (one launch per pass for EMBED and LM) at span S on
 * sequence 0's current cache, timed with HIP events around the passes on the
 * context stream (no commit).  The KV rows of positions p..p+S-1 are
 * rewritten, as a verify would. */
SPEC_API int spec_time_op(spec_ctx* ctx, int op, int S, int reps, float* us_per_launch);

/* The measured HBM read peak the roofline fractions are also reported
 * against: `reps` launches of a streaming-read kernel (16-byte non-temporal
 * loads, eight in flight per thread, 8 workgroups per CU) over the
 * caller-owned device buffer `buf` of `bytes` (>= 1 MiB, a multiple of 16;
 * much larger than the caches to measure HBM), timed with HIP events on
 * `hip_stream`; sink: 256 words of caller-owned device memory.
 * *gbps_out = bytes * reps / time. */
SPEC_API int spec_measure_read_bw(const void* buf, size_t bytes, uint32_t* sink, int reps, void* hip_stream,
                                  double* gbps_out);

/* The floor of a kernel-per-operation forward: n_regions back-to-back
 * launches of the same streaming-read kernel (grid workgroups of 256 threads,
 * 1..65535) over consecutive regions of region_bytes (>= 16, a multiple of
 * 16; 16 bytes is a launch with next to no work) of the caller-owned device
 * buffer buf, which must hold n_regions * region_bytes bytes (regions never
 * repeat, so with enough of them the reads come from HBM, not the caches).
 * The launches are captured once into a HIP graph on hip_stream (not the
 * null stream), replayed once untimed and once between HIP events; sink: 256
 * words of caller-owned device memory.  *us_out = the replay's time / n_regions. */
SPEC_API int spec_measure_read_chain(const void* buf, size_t region_bytes, int n_regions, int grid, uint32_t* sink,
                                     void* hip_stream, double* us_out);

/* Algorithmic bytes one launch of an op class streams at span S and cache
 * length ctx_len (weights, KV reads and writes; activations excluded). */
SPEC_API int spec_op_bytes(const spec_model_desc* desc, int op, int S, int ctx_len, double* bytes_out);

/* ----------------------------------------------------------- proposer */

/* n-gram prompt-lookup proposer (TensorSharp speculative decoding page,
 * n-gram section; coreai-model-zoo dense n-gram note, adaptive-K section):
 * an exact index per order n in [n_min, n_max] maps each n-gram to its most
 * recent end position, so propose() returns the continuation of the latest
 * earlier occurrence of the longest matching suffix, at most K tokens and
 * only tokens already in the history.  Host memory only. */
typedef struct spec_ngram spec_ngram;
SPEC_API int spec_ngram_create(int n_min, int n_max, int capacity, spec_ngram** out);
SPEC_API int spec_ngram_destroy(spec_ngram* ng);
SPEC_API int spec_ngram_append(spec_ngram* ng, const int32_t* toks, int n); /* ECAPACITY past capacity */
SPEC_API int spec_ngram_truncate(spec_ngram* ng, int len);
SPEC_API int spec_ngram_len(spec_ngram* ng);
/* Returns the number of drafts written (0..K), or a negative code. */
SPEC_API int spec_ngram_propose(spec_ngram* ng, int K, int32_t* drafts);

/* Adaptive K (coreai note, adaptive-K section): after a round that proposed
 * `drafted` >= 1 drafts of which `accepted` were accepted, K+2 on a full
 * accept, K-1 otherwise, clamped to [1, k_cap]; drafted == 0 returns k.
 * Pure function. */
SPEC_API int spec_adapt_k(int k, int drafted, int accepted, int k_cap);

/* ------------------------------------------------------ cost governor */

/* Speculation cost governor (TensorSharp speculative decoding page, protocol
 * section: speculation must never make decoding slower, so a governor times
 * speculative against plain steps at run time, parks drafting while it loses
 * and re-probes with backoff; the governor paragraphs give the numbers).
 * Host-only policy over the verify loop: before each step the caller asks
 * spec_governor_should_draft (1: speculate, 0: plain step), runs the step and
 * reports it with spec_governor_record.  A speculative step that drafted
 * nothing is still recorded as speculative (a one-token sample).  States:
 * baseline (plain steps measuring the plain cost), probe (speculative steps
 * measured against it), hold (speculating after a win, re-checked on the
 * last hold_window steps, baseline refreshed every hold_refresh steps),
 * parked (plain steps only).  NULL params give the page's numbers. */
typedef struct spec_governor spec_governor;
typedef struct spec_governor_params {
  int32_t probe_spec;       /* speculative steps of a full probe (8) */
  int32_t probe_spec_short; /* of a re-probe after a loss (3) */
  int32_t probe_plain;      /* plain steps measuring or refreshing the baseline (3) */
  int32_t park_first;       /* first park, in steps (32); doubles per loss ... */
  int32_t park_max;         /* ... up to this many (256) */
  int32_t zero_accept_exit; /* this many speculative steps in a row accepting nothing end a probe (4) */
  int32_t hold_window;      /* speculative steps averaged while a win holds (8) */
  int32_t hold_refresh;     /* held steps between baseline refreshes (64) */
} spec_governor_params;
typedef struct spec_governor_stats {
  int64_t wins, losses, probes;
  int64_t spec_steps, plain_samples, parked_steps;
  int32_t state;            /* 0 baseline, 1 probe, 2 hold, 3 parked */
  double plain_ms_per_token, spec_ms_per_token;
} spec_governor_stats;
SPEC_API int spec_governor_create(const spec_governor_params* params, spec_governor** out);
SPEC_API int spec_governor_destroy(spec_governor* g);
/* 1: the next step speculates; 0: it is a plain step (K = 0). */
SPEC_API int spec_governor_should_draft(spec_governor* g);
/* Report the step just run: speculative (must match the decision), tokens
 * committed (>= 1), drafts accepted, wall seconds of the whole step.
 * ESTATE if the step did not follow the decision. */
SPEC_API int spec_governor_record(spec_governor* g, int speculative, int committed, int accepted, double seconds);
/* A new request shares the governor: what is left of a park is capped at the
 * first park length and the backoff restarts there. */
SPEC_API int spec_governor_new_request(spec_governor* g);
SPEC_API int spec_governor_get_stats(spec_governor* g, spec_governor_stats* out);

/* ------------------------------------------------------ generation loop */

#define SPEC_DRAFT_NGRAM 0   /* n-gram proposer over prompt + committed tokens */
#define SPEC_DRAFT_STREAM 1  /* drafts read from `ref_stream` (perfect-draft bound) */
#define SPEC_DRAFT_WRONG 2   /* ref_stream tokens + 1 mod vocab (all-rejected bound) */

typedef struct spec_gen_params {
  int32_t spec;        /* 0: plain greedy, one K=0 step per token; 1: speculative */
  int32_t fixed_k;     /* > 0: fixed draft length; 0: adaptive K starting at 1 */
  int32_t k_cap;       /* cap of adaptive K (<= SPEC_MAX_SPAN-1) */
  int32_t n_min, n_max;
  int32_t draft_source;        /* SPEC_DRAFT_* */
  const int32_t* ref_stream;   /* [n_tokens] for SPEC_DRAFT_STREAM / WRONG */
  int32_t governed;            /* 1: a cost governor (default numbers) decides which steps draft */
} spec_gen_params;

typedef struct spec_gen_stats {
  int64_t forwards, drafted, accepted;
  int64_t accept_hist[SPEC_MAX_SPAN];           /* rounds by accepted drafts m */
  int64_t forwards_by_span[SPEC_MAX_SPAN + 1];  /* rounds by span length K+1 */
  double decode_s;  /* wall time from prefill return to the last token committed */
  double host_s;    /* part of decode_s spent outside spec_verify (proposer, bookkeeping) */
  double prefill_s;
  int64_t plain_steps;  /* steps the governor ran plain (parked or measuring the baseline) */
} spec_gen_stats;

/* Greedy generation on sequence 0: prefill `prompt`, then commit n_tokens
 * tokens counted from g0 (so decode covers n_tokens-1 committed after g0).
 * No round drafts past the budget.  out_tokens: [n_tokens]. */
SPEC_API int spec_generate(spec_ctx* ctx, const int32_t* prompt, int n_prompt, int n_tokens,
                  const spec_gen_params* params, int32_t* out_tokens, spec_gen_stats* stats);

/* The same loop in resumable form.  spec_gen_begin prefills `prompt` on
 * sequence 0 and commits g0 (budget: `capacity` committed tokens, g0
 * included; ref_stream, if used, must hold `capacity` tokens and outlive the
 * handle).  spec_gen_step runs up to `rounds` propose -> verify -> commit
 * rounds, stopping early at the budget, adds its counts and times to *stats
 * and returns the number of rounds run.  spec_gen_tokens copies the committed
 * tokens (up to cap) and returns how many there are. */
typedef struct spec_gen spec_gen;
SPEC_API int spec_gen_begin(spec_ctx* ctx, const int32_t* prompt, int n_prompt, int capacity,
                   const spec_gen_params* params, spec_gen** out);
SPEC_API int spec_gen_step(spec_gen* gen, int rounds, spec_gen_stats* stats);
SPEC_API int spec_gen_tokens(spec_gen* gen, int32_t* out, int cap);
/* The governor's counters of a governed loop (EINVAL if not governed). */
SPEC_API int spec_gen_governor_stats(spec_gen* gen, spec_governor_stats* out);
SPEC_API int spec_gen_end(spec_gen* gen);

#ifdef __cplusplus
}
#endif
#endif /* SPECV_H */
