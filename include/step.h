/* step.h - C ABI of libstep: one decode or mixed step of a dense decoder-only transformer
 * (RMSNorm, fused QKV with optional bias and per-head QK-norm, rotate-half RoPE, paged KV,
 * GQA attention, SwiGLU MLP, tied or untied LM head) on one AMD Instinct MI355X (gfx950).
 *
 * The method these calls implement is described on the pages:
 *   - "Removing overhead: fusion, graphs and async scheduling", sections "Fewer, larger matmuls"
 *     (stacked [W_Q | W_K | W_V] and [W_gate | W_up] projections, fused norm/activation) and
 *     "CUDA graphs for a changing batch" (one graph per batch-size bucket over static buffers,
 *     padding rows with slot -1 and length 0, eager fallback over the same buffers);
 *   - "Fast decode: syncs, CUDA graphs and compilation", sections "Sampling without the CPU"
 *     (Gumbel-max on the device), "Static shapes and a static cache" and "The fast decoder"
 *     (the step touches only static buffers and advances token and position in place);
 *   - "One forward per step", section "What changed" (prefill chunks first and decode rows last
 *     in one packed forward; attention splits by kind inside the call).
 *
 * Conventions
 *   - Every pointer named d_* is DEVICE memory; h_* is HOST memory. The caller owns all of it.
 *     The library borrows the pointers passed to step_init for the context's lifetime and
 *     allocates no device memory after step_init returns; it owns only the context, its
 *     graphs and a small pinned host staging area.
 *   - Matrices are row-major [out_features][in_features] in the model dtype.
 *   - The KV pools of each layer are in the model dtype, zero-filled by the caller. The K pool is
 *     [num_blocks][kv_heads][block_size][head_dim] (key-major); the V pool is
 *     [num_blocks][kv_heads][head_dim][block_size] (dim-major), so element (token t of a block,
 *     dim i) of a (block, kv head) tile is at t * head_dim + i in K and at i * block_size + t in V.
 *     Block num_blocks-1 is the scratch block: it must never appear in a block table; rows with
 *     slot -1 write there.
 *   - A token at absolute position p of a request whose block-table row is bt lives at slot
 *     bt[p / block_size] * block_size + p % block_size.
 *   - seq_len of a decode row counts the keys the row attends to INCLUDING its own token
 *     (cached + 1). A row with seq_len 0 is padding and produces a zero attention output.
 *   - Calls only enqueue work on the context's stream; nothing synchronises the stream except
 *     step_init (capture) and step_destroy. Outputs are valid once the stream reaches them.
 *   - Every function returns STEP_OK (0) or a negative error code and never throws; the
 *     message of the last error is in step_last_error(ctx).
 */
#ifndef GRAPH_REPLAY_AMD_STEP_H
#define GRAPH_REPLAY_AMD_STEP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  STEP_OK = 0,
  STEP_EINVAL = -1,        /* bad sizes, counts, pointers or a row count above the largest bucket */
  STEP_EUNSUPPORTED = -2,  /* a dtype / flag combination this build has no kernels for */
  STEP_EHIP = -3,          /* a HIP runtime call failed (message holds hipGetErrorString) */
  STEP_ECAPTURE = -4,      /* graph capture or instantiation failed */
  STEP_ESTATE = -5         /* call on a NULL or destroyed context */
};
enum { STEP_F32 = 0, STEP_BF16 = 1, STEP_F16 = 2 };
#define STEP_MAX_BUCKETS 16

typedef struct step_ctx step_ctx;

typedef struct {
  int32_t dtype;                 /* STEP_F32 / STEP_BF16 / STEP_F16: weights, KV pool, matmul inputs */
  int32_t layers, hidden, q_heads, kv_heads, head_dim, intermediate, vocab;
  int32_t qk_norm;               /* 1: per-head RMSNorm of q and k (one gain [head_dim] each) before RoPE */
  int32_t qkv_bias;              /* 1: bias [q_heads+2*kv_heads][head_dim] added after the QKV matmul */
  float rms_eps, rope_theta;
  int32_t block_size;            /* KV block size in tokens (16) */
  int32_t num_blocks;            /* blocks per layer pool, including the scratch block */
  int32_t max_blocks_per_seq;    /* block-table row width */
  int32_t max_position;          /* positions are in [0, max_position) */
  int32_t max_batch;             /* largest decode row count (== the largest bucket) */
  int32_t max_tokens;            /* largest packed token count of a mixed step (0: no mixed steps) */
  int32_t max_reqs;              /* largest request count of a mixed step */
  int32_t max_logit_rows;        /* largest number of sampled rows of a mixed step */
  int32_t num_buckets;           /* ascending decode batch sizes; the last must equal max_batch */
  int32_t buckets[STEP_MAX_BUCKETS];
  int32_t use_graphs;            /* 1: capture one hipGraph per bucket at init; 0: launch eagerly */
  /* Token-count buckets of mixed steps (ascending, each in [1, max_tokens]). With at least one, a
   * mixed step whose packed token count fits a bucket (and prefill_attention == 0) is padded to the
   * smallest such bucket and runs a launch plan that depends on the bucket only: padding tokens
   * (token 0, position 0, slot -1, no keys), a prefill tile list padded to bucket/16 + max_reqs,
   * decode-row attention over a device row list of max_reqs entries with splits sized for
   * max_position, and max_logit_rows logits rows of which the first num_logits are sampled. That
   * plan is captured as one hipGraph per bucket at init when use_graphs is 1 and launched eagerly
   * otherwise, with the same results. Larger steps, and steps with prefill_attention == 1, run the
   * exact-size eager plan. 0 buckets: every mixed step runs the exact-size eager plan. */
  int32_t num_mixed_buckets;
  int32_t mixed_buckets[STEP_MAX_BUCKETS];
  /* 1: decode and mixed steps apply per-row top-k / top-p filters before the Gumbel-max argmax (one
   * more kernel per step, captured in the graphs); 0: no filters, and the batches' h_top_k / h_top_p
   * must be NULL. "Fast decode: syncs, CUDA graphs and compilation", section "Sampling without the
   * CPU": filtered logits are set to -inf before the argmax; top-k with a fixed k, top-p as a sort
   * and a mask. Semantics (rows with T > 0 only, on z = logit / T in fp32): top-k keeps every z >=
   * the k-th largest z (k <= 0 or k >= vocab: off); top-p then keeps, in the order (z desc, index
   * asc), each token while the softmax mass (over the top-k set) before it is < p (p >= 1: off).
   * Top-p only looks at tokens within 30 of the largest z; a p that needs more keeps the whole
   * top-k set (the mass left out is below 2e-8). */
  int32_t sampling_filters;
  /* 1: decode steps of at most 8 rows append blocks to each layer's attention launch that load the
   * weights of the layer's O, gate|up and down projections into the L2 of the XCD whose GEMV blocks
   * will read them (HBM is otherwise idle during attention). A performance hint only: results are
   * the same bits either way. 0: off. */
  int32_t weight_prefetch;
  /* 1: decode steps of one row (bucket 1) run as ONE persistent kernel of one block per CU plus the
   * sampler, instead of about five kernels per layer: "Removing overhead: fusion, graphs and async
   * scheduling", section "Fewer, larger matmuls" (fewer, larger kernels) taken to a single launch,
   * "Fast decode: syncs, CUDA graphs and compilation", section "Where the time goes" (a batch-1 step
   * of ~600 small kernels is bound by their overhead, not by bandwidth). The phases of a layer hand
   * their outputs to the next through tagged device-memory words inside the kernel. Same results
   * as the multi-kernel step up to rounding order. Built for 16-bit dtypes at hidden 1024, 16 x 128
   * query dims, intermediate 3072, 2 query heads per KV head (Qwen3-0.6B's widths; up to 64 layers,
   * vocabulary >= 2048), max_position <= 128 * 256 / kv_heads (4,096 at those widths: one attention
   * split per block, of 64 keys up to 64 * 256 / kv_heads positions and of 128 keys beyond) and a
   * device of at least 256 CUs (one block each); other
   * configurations get STEP_EUNSUPPORTED at step_init. buckets[0] must be 1. Other buckets keep
   * the multi-kernel step. 0: off. */
  int32_t persistent_decode;
  /* Row attention launches over at least this many rows (16-bit K/V, at most 1,024 rows) run on the
   * balanced kernel, which cuts the launch's keys into equal shares per wave whatever the rows'
   * lengths; fewer rows use the split-KV grid. 0: the default, 128. Otherwise at least 9 (the split
   * grid keeps 8 rows and fewer); above 1,024: never. The balanced kernel's split points follow the
   * whole batch's lengths, so a row's output can change in its last bits with the other rows'
   * lengths (padding rows have none and change nothing); the split grid's follow the row and the
   * launch's key bound (max_position for decode steps and bucketed mixed steps, the step's longest
   * row in the exact-size mixed plan). */
  int32_t balanced_attention_rows;
} step_config;

typedef struct {
  const void *d_embed;           /* [vocab][hidden] */
  const void *d_lm_head;         /* [vocab][hidden]; equal to d_embed for tied embeddings */
  const void *d_final_norm;      /* [hidden] */
  /* host arrays of `layers` device pointers each */
  const void *const *d_in_norm;    /* [hidden] */
  const void *const *d_qkv_w;      /* [(q_heads+2*kv_heads)*head_dim][hidden]: rows of W_Q, then W_K, then W_V */
  const void *const *d_qkv_b;      /* [(q_heads+2*kv_heads)*head_dim] or NULL array when qkv_bias == 0 */
  const void *const *d_q_norm;     /* [head_dim] or NULL array when qk_norm == 0 */
  const void *const *d_k_norm;     /* [head_dim] or NULL array when qk_norm == 0 */
  const void *const *d_o_w;        /* [hidden][q_heads*head_dim] */
  const void *const *d_post_norm;  /* [hidden] */
  const void *const *d_gate_up_w;  /* [2*intermediate][hidden]: rows of W_gate, then W_up */
  const void *const *d_down_w;     /* [hidden][intermediate] */
} step_weights;

typedef struct {
  void *const *d_k_pool;         /* host array of `layers` device pointers (pool layout above) */
  void *const *d_v_pool;
  float *d_logits;               /* [max(max_batch, max_logit_rows)][vocab] fp32 output */
  int32_t *d_tokens;             /* [max(max_batch, max_logit_rows)] sampled token ids */
  int32_t *d_history;            /* optional [max_batch][max_position]: decode row b's sampled token is
                                    stored at [b][its input position]; NULL to skip */
  void *d_workspace;             /* >= step_workspace_bytes(cfg) bytes, 256-byte aligned */
  size_t workspace_bytes;
} step_buffers;

/* One decode step of r rows (host arrays of length r; block_table is r x bt_width). */
typedef struct {
  int32_t num_rows, bt_width;
  const int32_t *h_tokens, *h_positions, *h_seq_lens, *h_slot_mapping, *h_block_table;
  const float *h_temperature;    /* [num_rows]; NULL => all greedy; 0 => greedy row */
  uint64_t seed;                 /* Philox key for the Gumbel noise of this and later continued steps */
  const int32_t *h_top_k;        /* [num_rows] or NULL (off); needs sampling_filters; kept by continued steps */
  const float *h_top_p;          /* [num_rows] or NULL (off); needs sampling_filters; kept by continued steps */
} step_batch;

/* One packed mixed step: prefill requests first (their chunk tokens contiguous), decode requests
 * last (one token each). Host arrays. */
typedef struct {
  int32_t num_tokens, num_prefill_reqs, num_decode_reqs, num_logits, bt_width;
  const int32_t *h_query_start_loc;  /* [reqs+1] token offsets of each request in the packed sequence */
  const int32_t *h_seq_lens;         /* [reqs] keys after this step (cached + new tokens) */
  const int32_t *h_tokens, *h_positions, *h_slot_mapping;   /* [num_tokens] */
  const int32_t *h_block_table;      /* [reqs][bt_width] */
  const int32_t *h_logits_indices;   /* [num_logits] packed token rows whose logits are computed */
  const float *h_temperature;        /* [num_logits] or NULL (greedy) */
  uint64_t seed;
  int32_t prefill_attention;         /* 0: packed MFMA kernel (16-bit dtypes); 1: one query row per token */
  const int32_t *h_top_k;            /* [num_logits] or NULL (off); needs sampling_filters */
  const float *h_top_p;              /* [num_logits] or NULL (off); needs sampling_filters */
} step_packed;

/* Device bytes the workspace must hold for this configuration (0 if the configuration is invalid). */
size_t step_workspace_bytes(const step_config *cfg);

/* Validate, carve the workspace, build the RoPE table (fp64 angles rounded to fp32), zero the
 * scratch block, and capture one graph per bucket (largest first, after two warm-up runs) when
 * use_graphs is set. `stream` is a hipStream_t (NULL: the null stream). */
int step_init(const step_config *cfg, const step_weights *w, const step_buffers *b, void *stream,
              step_ctx **out);

/* Decode step over r = h_batch->num_rows rows. 1 <= r <= max_batch, bt_width <= max_blocks_per_seq,
 * else STEP_EINVAL. A row with seq_len > 0 must have seq_len == position + 1 and the slot its block
 * table gives for that position (STEP_EINVAL otherwise): its new K and V are written by the attention
 * kernel itself. The rows are copied into the static buffers and padded up to the smallest
 * bucket >= r (token 0, position 0, slot -1, seq_len 0, zero block-table row); the bucket's graph
 * is replayed (or its kernels launched eagerly). h_batch == NULL continues on the device: the
 * previous step's sampled tokens become the inputs, positions and seq_lens advance by one and the
 * slots are recomputed from the block table; the padded row count stays that of the last batch.
 * Logits rows [0, r) and tokens [0, r) are written. */
int step_decode(step_ctx *ctx, const step_batch *h_batch);

/* Mixed (or pure prefill) step, run eagerly: all tokens go through every layer once; prefill
 * attention is packed and causal per request, decode rows attend one query row per request; logits
 * and tokens are produced for h_logits_indices only (rows [0, num_logits) of the outputs). */
int step_mixed(step_ctx *ctx, const step_packed *h_batch);

/* Standalone sampler over d_logits [rows][ld] fp32: temperature h_temperature[row] (NULL: greedy);
 * optional per-row top-k h_top_k and top-p h_top_p (NULL: off; semantics as for sampling_filters,
 * which this call does not need); d_uniforms [rows][ld] fp32 supplies the uniforms (NULL:
 * Philox-4x32-10 keyed by seed with step counter `counter`). Writes d_tokens_out[rows]. */
int step_sample(step_ctx *ctx, const float *d_logits, int32_t rows, int32_t ld, int32_t vocab,
                const float *h_temperature, const int32_t *h_top_k, const float *h_top_p,
                const float *d_uniforms, uint64_t seed, uint64_t counter, int32_t *d_tokens_out);

/* Profiling (a debug aid, not part of the graphed path): runs one decode step at the bucket of the last
 * batch EAGERLY over the current static state, behind a short bounded device-side wait so the kernels
 * run back to back, launching every kernel with start/stop hipEvents that carry the dispatch's own
 * begin and end timestamps, and waits for it. Writes the execution time (ms) and the kind (see
 * step_kernel_kind_name) of up to max_kernels kernels into host arrays. Returns the number of kernels
 * of the step, or a negative code. It is a real step: the decode state advances exactly as in
 * step_decode(ctx, NULL). */
int step_profile_decode(step_ctx *ctx, int32_t max_kernels, float *h_ms, int32_t *h_kind);
const char *step_kernel_kind_name(int32_t kind);
/* Persistent decode only (persistent_decode = 1): waits for the context's stream, then reports
 * whether any wait inside a persistent decode step gave up since the last call (it bounds every
 * wait, so a step always ends). STEP_OK, or STEP_EHIP with the site in step_last_error; the flag is
 * cleared. Without persistent_decode it returns STEP_OK.
 * While the flag is set, every persistent step (the one whose wait gave up and every later one, in
 * graph replays too) ends with its outputs marked invalid instead of computed: logits row 0 is NaN,
 * token 0 is -1, and the row is not advanced (input id, position, seq_len, slot and history keep
 * their values), so a device-continued loop never feeds an invalid token forward. The same holds
 * for any sampled row with no candidate (every score NaN): token -1, no advance. */
int step_device_status(step_ctx *ctx);
/* Test aid for the failure contract above: waits for the context's stream and sets the persistent
 * step's give-up flag to `site` (> 0) as a wait that gave up would, so that every bounded wait of
 * the next steps ends at once and their outputs are marked invalid. STEP_EINVAL without
 * persistent_decode or for site <= 0. step_device_status reports and clears it. */
int step_set_device_status(step_ctx *ctx, int32_t site);
/* Host-only sizing query of the row attention's partial outputs ("Removing overhead: fusion,
 * graphs and async scheduling", section "CUDA graphs for a changing batch": a launch's shape is
 * fixed per row count, never chosen from the batch's contents). Returns the most partial slots
 * (each q_heads x (head_dim + 2) floats) one attention launch over `rows` rows with keys bounded by
 * max_len uses: rows x splits on the split-KV grid, and for a decode step on the balanced kernel
 * (16-bit K/V, balanced_attention_rows to 1,024 rows) rows + 2,048 x (q_heads / kv_heads) / q_heads
 * rounded up (2,048 waves), whatever the keys; the larger of the two where both can run. rows must lie in
 * [1, max(max_batch, max_tokens)] and max_len in [1, max_position]; STEP_EINVAL otherwise or for an
 * invalid config. Writes to *capacity (when not NULL, and whenever cfg is valid) the slots the
 * workspace of this config holds, which no launch's demand exceeds. */
int32_t step_attention_slots(const step_config *cfg, int32_t rows, int32_t max_len, int64_t *capacity);
/* Phase timestamps of the last step_profile_decode of a persistent single-row step, in
 * microseconds after the kernel's start (block 0's view; -1 where none was taken): slot 8 l + k for
 * layer l holds k = 1 QKV input normed, 2 attention items done, 3 merges done, 4 O input arrived,
 * 5 MLP input normed, 6 down input arrived; slot 8 L + 1 the final norm, 8 L + 2 the end. Writes
 * up to max_stamps values into h_us and returns the number of slots (0 if none were taken). */
int step_phase_stamps(const step_ctx *ctx, int32_t max_stamps, double *h_us);

/* Rows of the bucket the last decode step ran at, and kernels launched per decode step. */
int step_last_bucket(const step_ctx *ctx);
int step_kernels_per_decode(const step_ctx *ctx, int32_t bucket);
/* Token-count bucket the last mixed step was padded to (see step_config.mixed_buckets), or 0 when
 * it ran the exact-size eager plan. */
int step_last_mixed_bucket(const step_ctx *ctx);

const char *step_last_error(const step_ctx *ctx);
void step_destroy(step_ctx *ctx);

#ifdef __cplusplus
}
#endif
#endif
