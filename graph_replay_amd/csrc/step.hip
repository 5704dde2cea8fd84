// libstep: the C ABI declared in include/step.h.
//
// Host side of the decode / mixed step: validation, the workspace layout, the launch sequence of a
// step, one hipGraph per decode bucket ("Removing overhead: fusion, graphs and async scheduling",
// section "CUDA graphs for a changing batch": static buffers sized for the largest bucket, copy-in
// and padding before each replay, capture largest bucket first after two warm-ups, eager launch of
// the same kernels when no graph exists), and the eager packed mixed step ("One forward per step",
// section "What changed").
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "attention.h"
#include "common.h"
#include "gemm.h"
#include "persistent.h"
#include "prefill.h"
#include "sample.h"
#include "../../include/step.h"

using namespace gr;

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Layout {  // byte offsets into the workspace
  size_t dmeta, dmeta_bytes;          // decode static inputs: rng[2] | ids | pos | slot | len | temp | bt
  size_t mmeta, mmeta_bytes;          // mixed step inputs
  size_t rope_cos, rope_sin;
  size_t resid[2], h, qkv, q, attn_o, d_o, d_d, act;
  size_t attn_part, attn_cnt, samp_val, samp_idx, samp_cnt, samp_done, samp_temp, samp_rng;
  size_t samp_topk, samp_topp, samp_filt, samp_cand;
  // persistent decode step: per-layer pointers, tagged hand-off words, control words, stamps
  size_t p_lw, p_qkv, p_part, p_attn, p_o, p_act, p_down, p_ctl, p_stamps, p_cand;
  int p_splits;                       // attention splits per KV head the partial words hold
  size_t total;
  int TM, RM, LM;                     // token rows, requests, sampled rows the buffers hold
  size_t attn_slots;                  // (row, split) partial slots the attention partials hold
  int ksplit_max;                     // partial copies of split-K outputs
};

struct Launch;  // forward

}  // namespace

struct step_ctx {
  step_config cfg{};
  step_weights w{};
  std::vector<const void*> in_norm, qkv_w, qkv_b, q_norm, k_norm, o_w, post_norm, gate_up_w, down_w;
  std::vector<void*> k_pool, v_pool;
  float* logits = nullptr;
  int* tokens = nullptr;
  int* history = nullptr;
  char* ws = nullptr;
  Layout lay{};
  hipStream_t stream = nullptr;
  hipStream_t cap_stream = nullptr;
  // a mixed step's decode-row attention runs on side_stream beside the packed prefill attention
  // (fork_ev / join_ev order it after the QKV work and before the O projection)
  hipStream_t side_stream = nullptr;
  hipEvent_t fork_ev = nullptr, join_ev = nullptr;
  std::vector<hipGraph_t> graphs;
  std::vector<hipGraphExec_t> execs;
  std::vector<int> kernels_per_bucket;
  std::vector<hipGraph_t> mgraphs;              // per mixed token-count bucket
  std::vector<hipGraphExec_t> mexecs;
  std::vector<int> kernels_per_mbucket;
  int last_mixed_bucket = 0;                    // bucket of the last mixed step (0: exact-size plan)
  int last_bucket = 0;
  gr::L2Prefetch pf{};                // weights the next attention launch prefetches (pf.n == 0: none)
  int launches = 0;                   // kernels enqueued by the current plan run
  uint64_t step_count = 0;            // Philox step counter the next host-fed step starts from
  bool have_batch = false;
  // pinned staging (two slots each, reused after their copy has completed)
  char* h_stage[2] = {nullptr, nullptr};
  hipEvent_t stage_ev[2] = {nullptr, nullptr};
  int stage_next = 0;
  size_t stage_bytes = 0;
  // profiling: start/stop events of every launch while prof_on
  bool prof_on = false;
  std::vector<hipEvent_t> prof_ev, prof_ev_end;
  std::vector<int> prof_kind;
  // persistent single-row decode step (persistent_decode): blocks per launch (0: not in use),
  // whether the next launch records phase stamps, and the stamps of the last profiled step
  int p_nb = 0;
  bool p_stamp_next = false;
  std::vector<unsigned long long> p_stamps;
  std::string err;
  bool dead = false;
};

static const void* c_embed_of(step_ctx* ctx) { return ctx->w.d_embed; }
static const void* c_lm_head_of(step_ctx* ctx) { return ctx->w.d_lm_head; }
static const void* c_final_norm_of(step_ctx* ctx) { return ctx->w.d_final_norm; }

namespace {

int fail(step_ctx* c, int code, const char* fmt, ...) noexcept {
  if (c) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    try {
      c->err = buf;
    } catch (...) {
      // no memory for the message: the code still reports the failure
    }
  }
  return code;
}

#define HIPCHK(ctx, call)                                                                          \
  do {                                                                                             \
    hipError_t e_ = (call);                                                                        \
    if (e_ != hipSuccess) return fail((ctx), STEP_EHIP, "%s failed: %s", #call, hipGetErrorString(e_)); \
  } while (0)

int elem_bytes(int dtype) { return dtype == STEP_F32 ? 4 : 2; }

enum KernelKind {
  KK_QKV = 0, KK_QKV_POST, KK_ATTN, KK_O, KK_GATE_UP, KK_DOWN, KK_LM_HEAD, KK_NORM, KK_SAMPLE, KK_PREFILL_ATTN,
  KK_SAMPLE_FILTER, KK_PERSIST, KK_COUNT
};
const char* const kKindNames[KK_COUNT] = {"qkv_proj", "qknorm_rope_kvwrite", "attn_decode", "o_proj", "gate_up_silu",
                                          "down_proj", "lm_head", "add_rmsnorm", "sample", "attn_prefill",
                                          "sample_filter", "decode_step_persistent"};

// Called before every kernel launch: counts it and, while profiling, marks its start.
// Profile events for the next launch: set by pre_launch during a profile step, taken by launch().
struct ProfSlot {
  hipEvent_t start = nullptr, stop = nullptr;
};
thread_local ProfSlot g_prof_next;

void pre_launch(step_ctx* ctx, int kind) {
  if (ctx->prof_on && ctx->launches < static_cast<int>(ctx->prof_ev.size())) {
    g_prof_next = ProfSlot{ctx->prof_ev[ctx->launches], ctx->prof_ev_end[ctx->launches]};
    ctx->prof_kind[ctx->launches] = kind;
  }
  ctx->launches++;
}

// Every kernel of a step is launched here. During a profile step the launch carries start/stop
// events, which HIP stamps with the dispatch's own begin and end times (the kernel's execution,
// without the queueing around it); otherwise it is a plain launch, as captured into the graphs.
template <typename... KArgs, typename... Args>
void launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem, hipStream_t s, Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
  if (g_prof_next.start) {
    const ProfSlot p = g_prof_next;
    g_prof_next = ProfSlot{};
    hipExtLaunchKernelGGL(kernel, grid, block, static_cast<uint32_t>(shmem), s, p.start, p.stop, 0u,
                          static_cast<KArgs>(args)...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, shmem, s, static_cast<KArgs>(args)...);
  }
}

// A bounded wait on the device (about iters * 3.4 us) that lets the host queue a whole step behind
// it, so the profiled kernels run back to back.
__global__ void k_hold(int iters) {
  for (int i = 0; i < iters; ++i) __builtin_amdgcn_s_sleep(127);
}

// Keys per attention split for a row count and key bound (fixed per bucket, so the grid is too).
// Up to 8 rows, short splits fill the chip. Up to 64 rows whose contexts cannot pass 2,560 keys,
// one split per row in most cases: each extra split costs a block's fixed prologue and a merge,
// which measured more than the parallelism they buy (batch 32, contexts 128-2,048: 47.7 us at 512
// keys, 45.0 at 1,024, 44.4 at 2,048 per layer). Where rows can be longer, a few long rows would be
// the tail of the launch (32 decode rows with contexts up to 4,096 ran 7% slower at 2,048 keys), so
// they keep 512-key splits. From 256 keys up the length is then spread over the splits the bound
// needs, rounded up to whole 16-key blocks, so that no split holds only a few keys (a bound of
// 4,097 keys takes 8 splits of 528 rather than 9 of 512, the last with one key): batch 32 at
// 128-2,048 keys 2.201 against 2.234 ms per step.
int split_tokens_for(int rows, int max_len) {
  int P = rows <= 8 ? 64 : (rows <= 64 && max_len <= 2560 ? 2048 : 512);
  while ((max_len + P - 1) / P > gr::kMaxSplits) P *= 2;
  if (P >= 256) {
    const int n = std::max(1, max_len / P);
    P = ((max_len + n - 1) / n + gr::kBlk - 1) / gr::kBlk * gr::kBlk;
  }
  return P;
}

// Rows from which the balanced kernel (k_attn_flat) takes over from the split grid, for 16-bit
// K/V (step_config.balanced_attention_rows; 0 picks the default). Measured per layer on Qwen3-0.6B:
// 32 rows of 128-2,048 keys take 46 us on the split grid and 53 us balanced (each wave's share is
// then ~20 tiles, and the fixed costs of its pieces and merges outweigh the balance); 256 rows of
// 16-4,352 keys take 403 us on the split grid and 306 us balanced.
constexpr int kFlatMinRowsDefault = 128;
constexpr int kFlatMinRowsLeast = 9;   // at most 8 rows stay on the split grid (it carries the weight prefetch)
int flat_min_rows(const step_config& c) {
  return c.balanced_attention_rows > 0 ? c.balanced_attention_rows : kFlatMinRowsDefault;
}
bool use_flat(int rows, const step_config& c) {
  return c.dtype != STEP_F32 && rows >= flat_min_rows(c) && rows <= gr::kFlatMaxRows;
}

// Partial slots (each nq query heads of head_dim + 2 floats) that one attention launch over `rows`
// rows with keys bounded by max_len uses: a (row, split) pair each on the split grid; on the
// balanced kernel gr::flat_slots(rows, nkv) slots of G = nq / nkv heads.
size_t split_slot_demand(int rows, int max_len) {
  const int P = split_tokens_for(rows, max_len);
  return static_cast<size_t>(rows) * std::max(1, (max_len + P - 1) / P);
}
size_t flat_slot_demand(int rows, const step_config& c) {   // flat slots of G heads, in slots of nq heads
  const size_t G = static_cast<size_t>(c.q_heads / c.kv_heads);
  return (static_cast<size_t>(gr::flat_slots(rows, c.kv_heads)) * G + c.q_heads - 1) / c.q_heads;
}
// the most either kind of launch over `rows` rows uses (a decode step may run the balanced kernel,
// a mixed step's rows always run the split grid)
size_t attn_slot_demand(int rows, int max_len, const step_config& c) {
  const size_t sp = split_slot_demand(rows, max_len);
  return use_flat(rows, c) ? std::max(sp, flat_slot_demand(rows, c)) : sp;
}

// The most split-grid slots attention over `rows` rows may use at any key bound up to max_position.
// The split count is not monotone in the key bound (the split length doubles once a row would need
// more than kMaxSplits splits), so the bound uses the shortest split length any key bound can give
// this row count (512 keys stands for 2,048 where longer rows are possible) and caps it at
// kMaxSplits; spreading the length over the splits only ever lowers the count.
size_t split_slots_bound(int rows, int max_position) {
  const int P = rows <= 8 ? 64 : (rows <= 64 && max_position <= 2560 ? 2048 : 512);
  return static_cast<size_t>(rows) * std::min(gr::kMaxSplits, (max_position + P - 1) / P);
}

// copies of split-K partial outputs the workspace holds
constexpr int kMaxKsplit = 8;
// weight-prefetch blocks appended to an attention launch (about one per CU)
constexpr int kPrefetchBlocks = 256;

// 16-key tiles per compute wave and attention item of the persistent step: one (64-key items) while
// a row's items fit one per block, else two (128-key items)
int persist_tpw(const step_config& c) { return c.max_position <= 64 * gr::kPBlocks / c.kv_heads ? 1 : 2; }

bool compute_layout(const step_config& c, Layout& L) {
  const int H = c.hidden, d = c.head_dim, nq = c.q_heads, nkv = c.kv_heads, I = c.intermediate;
  const int QKV = (nq + 2 * nkv) * d;
  const int W = c.max_blocks_per_seq;
  const int MB = c.max_batch;
  L.TM = std::max(c.max_batch, c.max_tokens);
  L.RM = std::max(c.max_batch, c.max_reqs);
  L.LM = std::max(c.max_batch, c.max_logit_rows);
  const int TM = L.TM, RM = L.RM, LM = L.LM;
  const int eb = elem_bytes(c.dtype);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  // decode: rng[2] | ids | pos | slot | len | temp [MB] | bt [MB*W] | top_k | top_p [MB]
  L.dmeta_bytes = 16 + sizeof(int) * (7 * static_cast<size_t>(MB) + static_cast<size_t>(MB) * W);
  L.dmeta = take(L.dmeta_bytes);
  // mixed: rng[2] | tok | pos | slot | row_req | row_len [TM] | qsl [RM+1] | req_len [RM] | bt [RM*W]
  //        | logit_idx [LM] | temp [LM] | tile_req, tile_q0 [TM/16 + RM + 1] | dec_rows [RM] | n_logits
  //        | top_k [LM] | top_p [LM]
  const size_t tiles = TM / 16 + RM + 1;
  L.mmeta_bytes = 16 + sizeof(int) * (5 * static_cast<size_t>(TM) + (RM + 1) + RM + static_cast<size_t>(RM) * W +
                                      2 * static_cast<size_t>(LM) + 2 * tiles + RM + 1 + 2 * static_cast<size_t>(LM));
  L.mmeta = take(L.mmeta_bytes);
  L.rope_cos = take(sizeof(float) * static_cast<size_t>(c.max_position) * (d / 2));
  L.rope_sin = take(sizeof(float) * static_cast<size_t>(c.max_position) * (d / 2));
  L.ksplit_max = kMaxKsplit;
  L.resid[0] = take(sizeof(float) * static_cast<size_t>(TM) * H);
  L.resid[1] = take(sizeof(float) * static_cast<size_t>(TM) * H);
  L.h = take(static_cast<size_t>(eb) * TM * std::max(H, 1));
  L.qkv = take(sizeof(float) * static_cast<size_t>(kMaxKsplit) * TM * QKV);
  L.q = take(sizeof(float) * static_cast<size_t>(TM) * nq * d);
  L.attn_o = take(static_cast<size_t>(eb) * TM * nq * d);
  L.d_o = take(sizeof(float) * static_cast<size_t>(kMaxKsplit) * TM * H);
  L.d_d = take(sizeof(float) * static_cast<size_t>(kMaxKsplit) * TM * H);
  L.act = take(static_cast<size_t>(eb) * TM * I);
  // attention partials: the most slots any row count up to TM can use on the split grid (the bound
  // grows with the row count inside each split-length class, so the class's largest row count gives
  // its maximum), and on the balanced kernel (growing with the row count)
  size_t part_rows_splits = 0;
  for (int rows : {8, 64, TM}) part_rows_splits = std::max(part_rows_splits, split_slots_bound(std::min(rows, TM), c.max_position));
  const int flat_top = std::min(TM, gr::kFlatMaxRows);
  if (use_flat(flat_top, c)) part_rows_splits = std::max(part_rows_splits, flat_slot_demand(flat_top, c));
  L.attn_slots = part_rows_splits;
  L.attn_part = take(sizeof(float) * part_rows_splits * nq * (d + 2));
  L.attn_cnt = take(sizeof(unsigned) * static_cast<size_t>(TM) * nkv);
  const int nch_max = (c.vocab + 1023) / 1024;
  L.samp_val = take(sizeof(float) * static_cast<size_t>(LM) * nch_max);
  L.samp_idx = take(sizeof(int) * static_cast<size_t>(LM) * nch_max);
  L.samp_cnt = take(sizeof(unsigned) * static_cast<size_t>(LM));
  L.samp_done = take(sizeof(unsigned) * 4);
  // standalone sampler inputs: temperature | top_k | top_p [LM] each, one contiguous copy
  L.samp_temp = take(3 * sizeof(float) * static_cast<size_t>(LM));
  L.samp_topk = L.samp_temp + sizeof(float) * static_cast<size_t>(LM);
  L.samp_topp = L.samp_topk + sizeof(int) * static_cast<size_t>(LM);
  L.samp_filt = take(sizeof(uint2) * static_cast<size_t>(std::max(LM, MB)));
  // the LM head's fused sampler: one key per (block, row) of the streaming GEMV (<= 512 blocks, <= 48 rows)
  L.samp_cand = take(sizeof(unsigned long long) * 512 * 48);
  L.samp_rng = take(16);
  if (c.persistent_decode) {
    const int split = 64 * persist_tpw(c);
    L.p_splits = (c.max_position + split - 1) / split;
    L.p_lw = take(sizeof(gr::PLayer) * static_cast<size_t>(c.layers));
    L.p_qkv = take(sizeof(uint64_t) * static_cast<size_t>(QKV));
    L.p_part = take(sizeof(uint64_t) * static_cast<size_t>(nq) * L.p_splits * (d + 2));
    const size_t rep_bytes = sizeof(uint64_t) * static_cast<size_t>(gr::kPReplicas) * gr::kPRepStride;
    L.p_attn = take(rep_bytes);
    L.p_o = take(rep_bytes);
    L.p_act = take(rep_bytes);
    L.p_down = take(rep_bytes);
    L.p_ctl = take(4 * sizeof(unsigned));          // epoch | done | err | spare
    L.p_stamps = take(sizeof(unsigned long long) * gr::kPStamps);
    L.p_cand = take(sizeof(uint64_t) * gr::kPBlocks);
  }
  L.total = off;
  (void)RM;
  return true;
}

int validate_config(step_ctx* ctx, const step_config* c) {
  if (!c) return fail(ctx, STEP_EINVAL, "config is NULL");
  if (c->dtype != STEP_F32 && c->dtype != STEP_BF16 && c->dtype != STEP_F16)
    return fail(ctx, STEP_EUNSUPPORTED, "dtype %d is not one of F32/BF16/F16", c->dtype);
  if (c->layers <= 0 || c->hidden <= 0 || c->q_heads <= 0 || c->kv_heads <= 0 || c->intermediate <= 0 || c->vocab <= 0)
    return fail(ctx, STEP_EINVAL, "non-positive model dimension");
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(ctx, STEP_EUNSUPPORTED, "head_dim %d: kernels are built for 64 and 128", c->head_dim);
  if (c->q_heads % c->kv_heads != 0) return fail(ctx, STEP_EINVAL, "q_heads must be a multiple of kv_heads");
  const int G = c->q_heads / c->kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 6 && G != 8)
    return fail(ctx, STEP_EUNSUPPORTED, "query heads per KV head = %d: kernels are built for 1, 2, 4, 6, 8", G);
  const int epv = c->dtype == STEP_F32 ? 4 : 8;
  if (c->hidden % (c->dtype == STEP_F32 ? 4 : 32) || c->intermediate % 32 || (c->q_heads * c->head_dim) % 32)
    return fail(ctx, STEP_EUNSUPPORTED, "hidden, intermediate and q_heads*head_dim must be multiples of 32");
  (void)epv;
  if (c->hidden > 2048) return fail(ctx, STEP_EUNSUPPORTED, "hidden %d: norm kernels are built for <= 2048", c->hidden);
  if (c->block_size != 16) return fail(ctx, STEP_EUNSUPPORTED, "block_size must be 16");
  if (c->num_blocks < 2) return fail(ctx, STEP_EINVAL, "num_blocks must be >= 2 (one is the scratch block)");
  if (c->max_blocks_per_seq <= 0 || c->max_position <= 0) return fail(ctx, STEP_EINVAL, "bad max_blocks_per_seq / max_position");
  if (c->max_batch <= 0 || c->max_tokens < 0 || c->max_reqs < 0 || c->max_logit_rows < 0)
    return fail(ctx, STEP_EINVAL, "bad max_batch / max_tokens / max_reqs / max_logit_rows");
  if (c->num_buckets < 0 || c->num_buckets > STEP_MAX_BUCKETS) return fail(ctx, STEP_EINVAL, "num_buckets out of range");
  if (c->num_buckets == 0) return fail(ctx, STEP_EINVAL, "at least one bucket (== max_batch) is needed");
  for (int i = 0; i < c->num_buckets; ++i) {
    if (c->buckets[i] <= 0 || (i && c->buckets[i] <= c->buckets[i - 1]))
      return fail(ctx, STEP_EINVAL, "buckets must be positive and ascending");
  }
  if (c->buckets[c->num_buckets - 1] != c->max_batch) return fail(ctx, STEP_EINVAL, "last bucket must equal max_batch");
  if (c->max_tokens > 0 && (c->max_reqs <= 0 || c->max_logit_rows <= 0))
    return fail(ctx, STEP_EINVAL, "mixed steps need max_reqs and max_logit_rows");
  if (c->num_mixed_buckets < 0 || c->num_mixed_buckets > STEP_MAX_BUCKETS)
    return fail(ctx, STEP_EINVAL, "num_mixed_buckets out of range");
  if (c->num_mixed_buckets > 0 && c->max_tokens <= 0)
    return fail(ctx, STEP_EINVAL, "mixed buckets need mixed-step buffers (max_tokens > 0)");
  for (int i = 0; i < c->num_mixed_buckets; ++i) {
    if (c->mixed_buckets[i] <= 0 || c->mixed_buckets[i] > c->max_tokens ||
        (i && c->mixed_buckets[i] <= c->mixed_buckets[i - 1]))
      return fail(ctx, STEP_EINVAL, "mixed buckets must be ascending and in [1, max_tokens]");
  }
  if (c->persistent_decode != 0 && c->persistent_decode != 1) return fail(ctx, STEP_EINVAL, "persistent_decode must be 0 or 1");
  if (c->balanced_attention_rows != 0 && c->balanced_attention_rows < kFlatMinRowsLeast)
    return fail(ctx, STEP_EINVAL, "balanced_attention_rows %d: 0 or at least %d", c->balanced_attention_rows,
                kFlatMinRowsLeast);
  if (c->persistent_decode) {
    if (c->dtype == STEP_F32 || c->head_dim != 128 || c->hidden != 1024 || c->q_heads * c->head_dim != 2048 ||
        c->intermediate != 3072 || G != 2)
      return fail(ctx, STEP_EUNSUPPORTED,
                  "persistent_decode is built for 16-bit dtypes at hidden 1024, 16 x 128 query dims, intermediate "
                  "3072 and 2 query heads per KV head");
    if (c->layers > gr::kPMaxLayers)
      return fail(ctx, STEP_EUNSUPPORTED, "persistent_decode holds at most %d layers", gr::kPMaxLayers);
    const int max_keys = std::min(128 * gr::kPMaxSplits, 128 * gr::kPBlocks / c->kv_heads);
    if (c->max_position > max_keys)
      return fail(ctx, STEP_EUNSUPPORTED, "persistent_decode needs max_position <= %d", max_keys);
    if (c->buckets[0] != 1) return fail(ctx, STEP_EINVAL, "persistent_decode serves bucket 1, which the buckets must hold");
    // every LM-head wave owns at least one row and at most 128 (the fused sampler keeps two per lane)
    if (c->vocab < 8 * gr::kPBlocks || c->vocab > 128 * 8 * gr::kPBlocks)
      return fail(ctx, STEP_EUNSUPPORTED, "persistent_decode needs %d <= vocab <= %d", 8 * gr::kPBlocks,
                  128 * 8 * gr::kPBlocks);
  }
  return STEP_OK;
}

template <class T>
const typename T::S* tp(const void* p) { return static_cast<const typename T::S*>(p); }

// ------------------------------------------------------------------------------------------------
// linear-layer dispatch

struct Lin {
  int M, N, K;
  const void* W;
  const void* bias;
  const void* x;
  int epi;
  void* out;
  int ldo;
  // fused-norm prologue (M <= 8, or fp32)
  int norm = 0;
  const float* r_in = nullptr;
  const float* delta = nullptr;
  int n_delta = 0;
  size_t delta_stride = 0;
  const void* embed = nullptr;
  const int* tok = nullptr;
  float* r_out = nullptr;
  const void* gain = nullptr;
  float eps = 0.f;
  int kind = KK_QKV;
  int ksplit_ok = 0;          // output may be split into fp32 partials (consumer sums them)
  int* ksplit_used = nullptr; // out: partial count
  size_t split_stride = 0;
  // LM head: the sampler to fuse into the streaming GEMV when that kernel runs (sampled is then set)
  const SampleArgs* smp = nullptr;
  bool* sampled = nullptr;
};

template <class T, int MT, int ROWS, int U>
hipError_t launch_gemv_ru(const GemmArgs& a, int epi, dim3 grid, hipStream_t s) {
  launch((k_gemv<T, MT, ROWS, U>), grid, dim3(256), 0, s, a, epi);
  return hipGetLastError();
}

// (rows per wave, vectors per lane per row in flight): (1, 4|8), (2, 2|4), (4, 2), (8, 2)
template <class T, int MT>
hipError_t launch_gemv_mt(const GemmArgs& a, int epi, int rows_pw, int u, dim3 grid, hipStream_t s) {
  switch (rows_pw) {
    case 1: return u > 4 ? launch_gemv_ru<T, MT, 1, 8>(a, epi, grid, s) : launch_gemv_ru<T, MT, 1, 4>(a, epi, grid, s);
    case 2: return u > 2 ? launch_gemv_ru<T, MT, 2, 4>(a, epi, grid, s) : launch_gemv_ru<T, MT, 2, 2>(a, epi, grid, s);
    case 4: return launch_gemv_ru<T, MT, 4, 2>(a, epi, grid, s);
    default:
      if constexpr (MT < 8) return launch_gemv_ru<T, MT, 8, 2>(a, epi, grid, s);
      else return hipErrorInvalidValue;
  }
}

// K chunk the VALU GEMV stages in LDS (elements), as computed in the kernel
int gemv_kc(int MT, int eb) {
  const int epv = 16 / eb;
  return (32768 / (MT * eb)) / (64 * epv) * (64 * epv);
}

// Launch geometry of k_gemv: MT token rows per block row, rows_pw weight rows per wave (the largest
// that still gives >= 512 blocks), per_block weight rows per block (EPI_SILU: gate rows, each with
// its up row), u vectors per lane in flight; grid (nblk, ygrid), block x reading the weight rows
// [x * per_block, (x + 1) * per_block) (and the matching up rows).
struct GemvGeom { int MT, rows_pw, per_block, u, nblk, ygrid; };
GemvGeom gemv_geom(int M, int N, int K, int epi, int eb) {
  GemvGeom g{};
  g.MT = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : 8;
  g.ygrid = (M + g.MT - 1) / g.MT;
  g.rows_pw = (g.MT >= 8) ? 4 : 8;   // 8 x 8 accumulators would spill
  const int min_rows = (epi == EPI_SILU) ? 2 : 1;
  const int nvl = (std::min(K, gemv_kc(g.MT, eb)) / (16 / eb) + 63) / 64;   // vectors per lane per row
  auto per_block = [&](int rpw) { return 4 * ((epi == EPI_SILU) ? rpw / 2 : rpw); };
  while (g.rows_pw > min_rows) {
    if (static_cast<long>((N + per_block(g.rows_pw) - 1) / per_block(g.rows_pw)) * g.ygrid >= 512) break;
    g.rows_pw /= 2;
  }
  g.per_block = per_block(g.rows_pw);
  g.u = g.rows_pw == 1 ? (nvl > 4 ? 8 : 4) : g.rows_pw == 2 ? (nvl > 2 ? 4 : 2) : 2;
  g.nblk = (N + g.per_block - 1) / g.per_block;
  return g;
}

template <class T>
int run_linear(step_ctx* ctx, const Lin& l) {
  GemmArgs a{};
  a.M = l.M; a.N = l.N; a.K = l.K; a.W = l.W; a.bias = l.bias; a.x = l.x;
  a.norm = l.norm; a.r_in = l.r_in; a.delta = l.delta; a.n_delta = l.n_delta; a.delta_stride = l.delta_stride;
  a.embed = l.embed; a.tok = l.tok; a.r_out = l.r_out; a.gain = l.gain; a.eps = l.eps;
  a.out = l.out; a.ldo = l.ldo; a.ksplit = 1; a.out_split_stride = l.split_stride;
  if (l.ksplit_used) *l.ksplit_used = 1;
  hipStream_t s = ctx->stream;
  hipError_t e;
  const bool is_f32 = std::is_same<T, F32>::value;
  pre_launch(ctx, l.kind);
  if (l.M <= 8 || is_f32 || l.norm) {
    const int eb = static_cast<int>(sizeof(typename T::S));
    const GemvGeom g = gemv_geom(l.M, l.N, l.K, l.epi, eb);
    const int MT = g.MT;
    if (l.norm && (l.K > 2048 || l.K > gemv_kc(MT, eb))) e = hipErrorInvalidValue;   // one-chunk prologue only
    dim3 grid(g.nblk, g.ygrid);
    if (!(l.norm && (l.K > 2048 || l.K > gemv_kc(MT, eb)))) switch (MT) {
      case 1: e = launch_gemv_mt<T, 1>(a, l.epi, g.rows_pw, g.u, grid, s); break;
      case 2: e = launch_gemv_mt<T, 2>(a, l.epi, g.rows_pw, g.u, grid, s); break;
      case 4: e = launch_gemv_mt<T, 4>(a, l.epi, g.rows_pw, g.u, grid, s); break;
      default: e = launch_gemv_mt<T, 8>(a, l.epi, g.rows_pw, g.u, grid, s); break;
    }
  } else if constexpr (!std::is_same<T, F32>::value) {
    constexpr int SW = 8, SC = 8;   // waves per block, k-steps per weight chunk
    if (l.kind == KK_LM_HEAD && l.M > 8 && !l.bias && l.epi == EPI_F32 && l.K % (32 * SC) == 0 &&
        ((l.M <= 32 && l.K <= 1024) || (l.M <= 48 && l.K <= 1536))) {
      // the vocabulary-wide output, each wave streaming whole weight tiles: two blocks per CU up
      // to 32 rows of K <= 1,024 (64 KiB of LDS each), else one (up to 48 rows of K <= 1,536)
      const int ntiles = (l.N + 15) / 16;
      const int per_cu = (l.M <= 32 && l.K <= 1024) ? 2 : 1;
      const dim3 grid(std::min(per_cu * 256, (ntiles + SW - 1) / SW));
      if (l.smp) {
        // the sampler in the epilogue (no separate sampling launch follows)
        a.smp = *l.smp;
        a.cand = reinterpret_cast<unsigned long long*>(ctx->ws + ctx->lay.samp_cand);
        a.cand_done = reinterpret_cast<unsigned*>(ctx->ws + ctx->lay.samp_done) + 1;
        if (l.sampled) *l.sampled = true;
        if (per_cu == 1) launch((gr::k_gemv_stream<T, 3, SW, SC, 1536, true>), grid, dim3(64 * SW), 0, s, a);
        else if (l.M <= 16) launch((gr::k_gemv_stream<T, 1, SW, SC, 1024, true>), grid, dim3(64 * SW), 0, s, a);
        else launch((gr::k_gemv_stream<T, 2, SW, SC, 1024, true>), grid, dim3(64 * SW), 0, s, a);
      } else {
        if (per_cu == 1) launch((gr::k_gemv_stream<T, 3, SW, SC, 1536, false>), grid, dim3(64 * SW), 0, s, a);
        else if (l.M <= 16) launch((gr::k_gemv_stream<T, 1, SW, SC, 1024, false>), grid, dim3(64 * SW), 0, s, a);
        else launch((gr::k_gemv_stream<T, 2, SW, SC, 1024, false>), grid, dim3(64 * SW), 0, s, a);
      }
      e = hipGetLastError();
    } else if (l.M <= 32) {
      // two 16-row weight tiles per wave share each activation fragment where the output is wide
      // enough (QKV, gate|up); narrow outputs (O, down) keep one tile and split K instead
      const int rt = (l.M > 16 && l.N >= 2048) ? 2 : 1;
      const int bx = (l.epi == EPI_SILU) ? (l.N + 8 * rt - 1) / (8 * rt) : (l.N + 16 * rt - 1) / (16 * rt);
      int ks = 1;
      if (l.ksplit_ok && l.epi == EPI_F32) {
        const int target = 256;
        while (ks < kMaxKsplit && bx * ks < target && (l.K / 32) / (ks * 2) >= 2) ks *= 2;
      }
      a.ksplit = ks;
      if (l.ksplit_used) *l.ksplit_used = ks;
      dim3 grid(bx, ks);
      if (l.M <= 16) launch((k_gemv_mfma<T, 1, 4, 1>), grid, dim3(256), 0, s, a, l.epi);
      else if (rt == 2) launch((k_gemv_mfma<T, 2, 4, 2>), grid, dim3(256), 0, s, a, l.epi);
      else launch((k_gemv_mfma<T, 2, 4, 1>), grid, dim3(256), 0, s, a, l.epi);
      e = hipGetLastError();
    } else if (l.K % 64 == 0 && l.ldo % 4 == 0) {
      // ring GEMM: gate|up on 128x128 tiles, other projections on 64x128 tiles with K split (fp32
      // partials) while the grid has fewer than 256 blocks and each split keeps >= 8 k-steps
      const bool silu_epi = l.epi == EPI_SILU;
      const int BN = silu_epi ? 128 : 64, BM = 128;
      const int n_tiles = silu_epi ? (l.N + BN / 2 - 1) / (BN / 2) : (l.N + BN - 1) / BN;
      const int m_tiles = (l.M + BM - 1) / BM;
      int ks = 1;
      if (l.ksplit_ok && l.epi == EPI_F32) {
        while (ks < kMaxKsplit && n_tiles * m_tiles * ks < 256 && (l.K / 64) / (ks * 2) >= 8) ks *= 2;
      }
      a.ksplit = ks;
      if (l.ksplit_used) *l.ksplit_used = ks;
      dim3 grid(8 * ((n_tiles + 7) / 8) * m_tiles, 1, ks);
      if (silu_epi && l.M > 256) {
        // many tokens: 256 x 192 tiles on 8 waves (110 FLOP per byte staged into LDS against 64 for
        // 128 x 128; the 544-token mixed step runs 3.5% faster)
        const int nt2 = (l.N + 127) / 128, mt2 = (l.M + 191) / 192;
        launch((k_gemm_ring<T, 256, 192, 4, 2, 2>), dim3(8 * ((nt2 + 7) / 8) * mt2), dim3(512), 0, s, a, l.epi, nt2, mt2);
      } else if (silu_epi) {
        launch((k_gemm_ring<T, 128, 128, 2, 2, 2>), grid, dim3(256), 0, s, a, l.epi, n_tiles, m_tiles);
      } else {
        launch((k_gemm_ring<T, 64, 128, 2, 2, 2>), grid, dim3(256), 0, s, a, l.epi, n_tiles, m_tiles);
      }
      e = hipGetLastError();
    } else {
      const bool big = l.M > 64;
      const int BN = big ? 128 : 64, BM = big ? 128 : 64;
      const int bx = (l.epi == EPI_SILU) ? (l.N + BN / 2 - 1) / (BN / 2) : (l.N + BN - 1) / BN;
      const int by = (l.M + BM - 1) / BM;
      int ks = 1;
      if (l.ksplit_ok && l.epi == EPI_F32) {
        while (ks < kMaxKsplit && bx * by * ks < 256 && (l.K / 32) / (ks * 2) >= 4) ks *= 2;
      }
      a.ksplit = ks;
      if (l.ksplit_used) *l.ksplit_used = ks;
      dim3 grid(bx, by, ks);
      if (big) launch((k_gemm<T, 128, 128>), grid, dim3(256), 0, s, a, l.epi);
      else launch((k_gemm<T, 64, 64>), grid, dim3(256), 0, s, a, l.epi);
      e = hipGetLastError();
    }
  } else {
    e = hipErrorInvalidValue;
  }
  if (e != hipSuccess) return fail(ctx, STEP_EHIP, "linear launch failed: %s", hipGetErrorString(e));
  return STEP_OK;
}

template <class T>
int run_norm(step_ctx* ctx, int M, const float* r_in, const float* delta, int n_delta, size_t dstride,
             const void* embed, const int* tok, const int* row_map, float* r_out, const void* gain, void* h_out) {
  const int H = ctx->cfg.hidden;
  pre_launch(ctx, KK_NORM);
  launch((k_add_rmsnorm<T>), dim3(M), dim3(256), 0, ctx->stream, H, r_in, delta, n_delta, dstride, embed,
                     tok, row_map, r_out, gain, h_out, ctx->cfg.rms_eps);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ctx, STEP_EHIP, "norm launch failed: %s", hipGetErrorString(e));
  return STEP_OK;
}

// fp32 K/V: FMA kernel; 16-bit K/V: matrix-core kernel, two blocks per wave step for long splits,
// or (flat_rows > 0) the balanced kernel over flat_rows grid rows
template <class T, int D, int G>
void launch_attn_rows_g(const AttnRowsArgs& a, dim3 grid, hipStream_t s, int flat_rows) {
  if constexpr (std::is_same<T, F32>::value) {
    launch((k_attn_rows<T, D, G>), grid, dim3(256), 0, s, a);
  } else {
    if (flat_rows > 0) launch((k_attn_flat<T, D, G, 2>), dim3(gr::kFlatBlocks), dim3(256), 0, s, a, flat_rows);
    else if (a.split_tokens >= 256) launch((k_attn_rows_mfma<T, D, G, 2>), grid, dim3(256), 0, s, a);
    else launch((k_attn_rows_mfma<T, D, G, 1>), grid, dim3(256), 0, s, a);
  }
}
template <class T, int D>
hipError_t launch_attn_rows_d(const AttnRowsArgs& a, int G, dim3 grid, hipStream_t s, int flat_rows) {
  switch (G) {
    case 1: launch_attn_rows_g<T, D, 1>(a, grid, s, flat_rows); break;
    case 2: launch_attn_rows_g<T, D, 2>(a, grid, s, flat_rows); break;
    case 4: launch_attn_rows_g<T, D, 4>(a, grid, s, flat_rows); break;
    case 6: launch_attn_rows_g<T, D, 6>(a, grid, s, flat_rows); break;
    default: launch_attn_rows_g<T, D, 8>(a, grid, s, flat_rows); break;
  }
  return hipGetLastError();
}

// Row attention over `rows` query rows; max_len bounds the keys of any row (sets the split grid).
// q == nullptr: decode rows, whose QK-norm + RoPE + KV write run inside the attention kernel from
// the n_qkv fp32 partial outputs of the QKV projection.
template <class T>
int run_attn_rows(step_ctx* ctx, int layer, int rows, const float* q, int n_qkv, const int* pos, const int* slot,
                  const int* bt, int bt_stride, const int* row_req, const int* seq_lens, int max_len, void* out,
                  const int* row_ids = nullptr) {
  const step_config& c = ctx->cfg;
  const Layout& Ly = ctx->lay;
  AttnRowsArgs a{};
  a.nq = c.q_heads; a.nkv = c.kv_heads; a.q = q;
  a.qkv = reinterpret_cast<const float*>(ctx->ws + Ly.qkv);
  a.n_parts = n_qkv;
  a.part_stride = static_cast<size_t>(Ly.TM) * (c.q_heads + 2 * c.kv_heads) * c.head_dim;
  a.pos = pos; a.slot = slot;
  a.rope_cos = reinterpret_cast<const float*>(ctx->ws + Ly.rope_cos);
  a.rope_sin = reinterpret_cast<const float*>(ctx->ws + Ly.rope_sin);
  a.q_norm = c.qk_norm ? ctx->q_norm[layer] : nullptr;
  a.k_norm = c.qk_norm ? ctx->k_norm[layer] : nullptr;
  a.eps = c.rms_eps;
  a.k_pool = ctx->k_pool[layer]; a.v_pool = ctx->v_pool[layer];
  a.block_table = bt; a.bt_stride = bt_stride; a.row_ids = row_ids; a.row_req = row_req; a.seq_lens = seq_lens;
  // The balanced kernel serves decode steps only (the fused prologue, one row per request): the
  // mixed step's decode rows run beside the packed prefill attention, where the split grid's launch,
  // sized by the rows, shares the GPU better (a 512-token chunk + 32 decode rows: 4.69 ms per step
  // on the split grid, 5.35 ms with the balanced kernel).
  const bool flat = q == nullptr && row_ids == nullptr && row_req == nullptr && use_flat(rows, c);
  a.split_tokens = split_tokens_for(rows, max_len);
  a.max_splits = flat ? 1 : std::max(1, (max_len + a.split_tokens - 1) / a.split_tokens);
  a.num_blocks = c.num_blocks;
  a.out = out;
  a.partials = reinterpret_cast<float*>(ctx->ws + Ly.attn_part);
  a.split_cnt = reinterpret_cast<unsigned*>(ctx->ws + Ly.attn_cnt);
  a.scale = 1.0f / sqrtf(static_cast<float>(c.head_dim));
  const int G = c.q_heads / c.kv_heads;
  if (rows > Ly.TM) return fail(ctx, STEP_EINVAL, "attention over %d rows exceeds the workspace's %d", rows, Ly.TM);
  if ((flat ? flat_slot_demand(rows, c) : split_slot_demand(rows, max_len)) > Ly.attn_slots)
    return fail(ctx, STEP_EINVAL, "attention over %d rows x %d splits exceeds the workspace's %zu partial slots", rows,
                a.max_splits, Ly.attn_slots);
  dim3 grid(rows, c.kv_heads, a.max_splits);
  if (ctx->pf.n > 0 && !flat) {
    a.pf = ctx->pf;
    const int plane = rows * c.kv_heads;
    grid.z += (kPrefetchBlocks + plane - 1) / plane;
  }
  pre_launch(ctx, KK_ATTN);
  const int flat_rows = flat ? rows : 0;
  hipError_t e = (c.head_dim == 64) ? launch_attn_rows_d<T, 64>(a, G, grid, ctx->stream, flat_rows)
                                    : launch_attn_rows_d<T, 128>(a, G, grid, ctx->stream, flat_rows);
  if (e != hipSuccess) return fail(ctx, STEP_EHIP, "attention launch failed: %s", hipGetErrorString(e));
  return STEP_OK;
}

template <class T>
int run_qkv_post(step_ctx* ctx, int layer, int rows, int n_parts, size_t part_stride, const int* pos, const int* slot) {
  const step_config& c = ctx->cfg;
  const Layout& L = ctx->lay;
  pre_launch(ctx, KK_QKV_POST);
  launch((k_qkv_post<T>), dim3(rows, c.q_heads + c.kv_heads), dim3(64), 0, ctx->stream, c.q_heads,
                     c.kv_heads, c.head_dim, reinterpret_cast<const float*>(ctx->ws + L.qkv), n_parts, part_stride, pos,
                     slot, reinterpret_cast<const float*>(ctx->ws + L.rope_cos),
                     reinterpret_cast<const float*>(ctx->ws + L.rope_sin), c.qk_norm ? ctx->q_norm[layer] : nullptr,
                     c.qk_norm ? ctx->k_norm[layer] : nullptr, c.rms_eps, reinterpret_cast<float*>(ctx->ws + L.q),
                     ctx->k_pool[layer], ctx->v_pool[layer], c.num_blocks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ctx, STEP_EHIP, "qkv_post launch failed: %s", hipGetErrorString(e));
  return STEP_OK;
}

// the sampler's arguments, shared by k_sample and the LM head's fused sampler
SampleArgs sample_args(step_ctx* ctx, const float* logits, int ld, int vocab, const float* temp, const float* uniforms,
                       const uint64_t* rng, uint64_t seed, uint64_t stepc, int* tokens_out, int advance, int* ids,
                       int* pos, int* lens, int* slots, const int* bt, int bt_stride, int* history, int hist_ld,
                       const int* n_rows, const int* halt) {
  SampleArgs a{};
  a.logits = logits; a.ld = ld; a.vocab = vocab;
  a.temperature = temp; a.uniforms = uniforms; a.rng = rng; a.seed = seed; a.step = stepc;
  a.part_val = reinterpret_cast<float*>(ctx->ws + ctx->lay.samp_val);
  a.part_idx = reinterpret_cast<int*>(ctx->ws + ctx->lay.samp_idx);
  a.row_cnt = reinterpret_cast<unsigned*>(ctx->ws + ctx->lay.samp_cnt);
  a.done_cnt = reinterpret_cast<unsigned*>(ctx->ws + ctx->lay.samp_done);
  a.tokens_out = tokens_out;
  a.advance = advance; a.input_ids = ids; a.positions = pos; a.seq_lens = lens; a.slots = slots;
  a.block_table = bt; a.bt_stride = bt_stride; a.history = history; a.hist_ld = hist_ld;
  a.n_rows = n_rows;
  a.halt = halt;
  return a;
}

int run_sample(step_ctx* ctx, const float* logits, int rows, int ld, int vocab, const float* temp, const float* uniforms,
               const uint64_t* rng, uint64_t seed, uint64_t stepc, int* tokens_out, int advance, int* ids, int* pos,
               int* lens, int* slots, const int* bt, int bt_stride, int* history, int hist_ld,
               const int* n_rows = nullptr, const int* topk = nullptr, const float* topp = nullptr,
               const int* halt = nullptr) {
  uint2* filt = nullptr;
  if (temp && (topk || topp)) {
    // per-row top-k / top-p cut first (one block of 1024 threads per row)
    FilterArgs f{};
    f.logits = logits; f.ld = ld; f.vocab = vocab; f.temperature = temp; f.top_k = topk; f.top_p = topp;
    f.n_rows = n_rows;
    f.filt = filt = reinterpret_cast<uint2*>(ctx->ws + ctx->lay.samp_filt);
    pre_launch(ctx, KK_SAMPLE_FILTER);
    launch(k_sample_filter, dim3(rows), dim3(kFilterThreads), 0, ctx->stream, f);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(ctx, STEP_EHIP, "sample filter launch failed: %s", hipGetErrorString(e));
  }
  SampleArgs a = sample_args(ctx, logits, ld, vocab, temp, uniforms, rng, seed, stepc, tokens_out, advance, ids, pos,
                             lens, slots, bt, bt_stride, history, hist_ld, n_rows, halt);
  // one or two 1,024-column passes per thread while the grid stays within 4,096 blocks: a thread's
  // passes are serial memory round trips, so short chunks finish sooner
  int chunk = 1024;
  while (chunk < 16384 && static_cast<long>(rows) * ((vocab + chunk - 1) / chunk) > 4096) chunk *= 2;
  a.chunk = chunk;
  a.filt = filt;
  const int nch = (vocab + chunk - 1) / chunk;
  pre_launch(ctx, KK_SAMPLE);
  launch(k_sample, dim3(rows, nch), dim3(256), 0, ctx->stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ctx, STEP_EHIP, "sample launch failed: %s", hipGetErrorString(e));
  return STEP_OK;
}

#define TRY(x)                  \
  do {                          \
    int rc_ = (x);              \
    if (rc_ != STEP_OK) return rc_; \
  } while (0)

// Pointers into a metadata block laid out as rng[2] | ids | pos | slot | len | temp | bt.
struct DecodeMeta {
  uint64_t* rng;
  int *ids, *pos, *slot, *len;
  float* temp;
  int* bt;
  int* topk;
  float* topp;
};
DecodeMeta decode_meta(char* base, int MB, int W) {
  DecodeMeta m;
  m.rng = reinterpret_cast<uint64_t*>(base);
  m.ids = reinterpret_cast<int*>(base + 16);
  m.pos = m.ids + MB;
  m.slot = m.pos + MB;
  m.len = m.slot + MB;
  m.temp = reinterpret_cast<float*>(m.len + MB);
  m.bt = reinterpret_cast<int*>(m.temp + MB);
  m.topk = m.bt + static_cast<size_t>(MB) * W;
  m.topp = reinterpret_cast<float*>(m.topk + MB);
  return m;
}

// The transformer layers over M rows: embed -> layers -> final norm (rows of row_map) -> LM head.
// attn(layer) enqueues the attention of one layer (rows or packed prefill + rows).
// fused_rope: the attention kernel does QK-norm + RoPE + KV write itself (decode rows, one token per
// request); otherwise k_qkv_post runs first so every chunk token's K and V are in the pool.
// Prefetch targets of layer l's attention launch: the gate|up, down and O GEMVs that follow it, as
// k_gemv lays them out for M rows (one block row: M <= 8).
template <class T>
void set_prefetch(step_ctx* ctx, int l, int M) {
  const step_config& c = ctx->cfg;
  const int eb = static_cast<int>(sizeof(typename T::S));
  const int H = c.hidden, I = c.intermediate, QD = c.q_heads * c.head_dim;
  struct Tg { const void* w; int N, K, epi; } tg[gr::kPrefetchTargets] = {
      {ctx->gate_up_w[l], I, H, EPI_SILU}, {ctx->down_w[l], H, I, EPI_F32}, {ctx->o_w[l], H, QD, EPI_F32}};
  gr::L2Prefetch& p = ctx->pf;
  p = gr::L2Prefetch{};
  for (int t = 0; t < gr::kPrefetchTargets; ++t) {
    const GemvGeom g = gemv_geom(M, tg[t].N, tg[t].K, tg[t].epi, eb);
    p.base[t] = static_cast<const char*>(tg[t].w);
    p.row_bytes[t] = tg[t].K * eb;
    p.pb[t] = g.per_block;
    p.n_rows[t] = tg[t].N;
    p.up_off[t] = (tg[t].epi == EPI_SILU) ? tg[t].N : 0;
    p.nblk[t] = g.nblk;
  }
  p.n = gr::kPrefetchTargets;
}

template <class T, class AttnFn>
int run_layers(step_ctx* ctx, int M, const int* tok, const int* pos, const int* slot, int n_logits, const int* logit_rows,
               bool fused_rope, AttnFn attn, const SampleArgs* smp = nullptr, bool* sampled = nullptr) {
  const step_config& c = ctx->cfg;
  const Layout& L = ctx->lay;
  const int H = c.hidden, d = c.head_dim, nq = c.q_heads, nkv = c.kv_heads, I = c.intermediate;
  const int QKV = (nq + 2 * nkv) * d;
  float* resid[2] = {reinterpret_cast<float*>(ctx->ws + L.resid[0]), reinterpret_cast<float*>(ctx->ws + L.resid[1])};
  void* h = ctx->ws + L.h;
  float* qkv = reinterpret_cast<float*>(ctx->ws + L.qkv);
  void* attn_o = ctx->ws + L.attn_o;
  float* d_o = reinterpret_cast<float*>(ctx->ws + L.d_o);
  float* d_d = reinterpret_cast<float*>(ctx->ws + L.d_d);
  void* act = ctx->ws + L.act;
  const int MT = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : 8;
  const bool fuse_norm = ((M <= 8) || std::is_same<T, F32>::value) && H <= 2048 &&
                         H <= gemv_kc(MT, static_cast<int>(sizeof(typename T::S)));
  const size_t res_stride = static_cast<size_t>(L.TM) * H;     // floats between split-K partials of H-wide outputs
  const size_t qkv_stride = static_cast<size_t>(L.TM) * QKV;
  int n_dd = 0;                                                 // partial count of the previous down output
  for (int l = 0; l < c.layers; ++l) {
    // ---- attention half: r1 = r0 + down(l-1); h = RMSNorm(r1) * in_norm; qkv = h Wqkv^T (+b)
    const float* r_in = resid[0];
    float* r_out = resid[1];
    const bool first = (l == 0);
    int n_qkv = 1;
    Lin lin{};
    lin.M = M; lin.N = QKV; lin.K = H; lin.W = ctx->qkv_w[l]; lin.bias = c.qkv_bias ? ctx->qkv_b[l] : nullptr;
    lin.epi = EPI_F32; lin.out = qkv; lin.ldo = QKV; lin.ksplit_ok = 1; lin.ksplit_used = &n_qkv; lin.kind = KK_QKV;
    lin.split_stride = qkv_stride;
    if (fuse_norm) {
      lin.norm = 1; lin.r_in = r_in; lin.delta = first ? nullptr : d_d; lin.n_delta = first ? 0 : n_dd;
      lin.delta_stride = res_stride; lin.embed = first ? c_embed_of(ctx) : nullptr; lin.tok = tok; lin.r_out = r_out;
      lin.gain = ctx->in_norm[l]; lin.eps = c.rms_eps;
    } else {
      TRY(run_norm<T>(ctx, M, r_in, first ? nullptr : d_d, first ? 0 : n_dd, res_stride, first ? c_embed_of(ctx) : nullptr,
                      tok, nullptr, r_out, ctx->in_norm[l], h));
      lin.x = h;
    }
    TRY(run_linear<T>(ctx, lin));
    if (!fused_rope) TRY(run_qkv_post<T>(ctx, l, M, n_qkv, qkv_stride, pos, slot));
    // decode rows: the attention launch also pulls this layer's remaining weights into L2
    if (fused_rope && c.weight_prefetch && M <= 8) set_prefetch<T>(ctx, l, M);
    const int ar = attn(l, n_qkv);
    ctx->pf.n = 0;
    TRY(ar);
    // ---- O projection
    int n_o = 1;
    Lin lo{};
    lo.M = M; lo.N = H; lo.K = nq * d; lo.W = ctx->o_w[l]; lo.x = attn_o; lo.epi = EPI_F32; lo.out = d_o; lo.ldo = H;
    lo.ksplit_ok = 1; lo.ksplit_used = &n_o; lo.split_stride = res_stride; lo.kind = KK_O;
    TRY(run_linear<T>(ctx, lo));
    // ---- MLP half: r0 = r1 + o; h = RMSNorm(r0) * post_norm; a = SiLU(h Wg^T) * (h Wu^T); down
    Lin lg{};
    lg.M = M; lg.N = I; lg.K = H; lg.W = ctx->gate_up_w[l]; lg.epi = EPI_SILU; lg.out = act; lg.ldo = I;
    lg.kind = KK_GATE_UP;
    if (fuse_norm) {
      lg.norm = 1; lg.r_in = r_out; lg.delta = d_o; lg.n_delta = n_o; lg.delta_stride = res_stride; lg.r_out = resid[0];
      lg.gain = ctx->post_norm[l]; lg.eps = c.rms_eps;
    } else {
      TRY(run_norm<T>(ctx, M, r_out, d_o, n_o, res_stride, nullptr, nullptr, nullptr, resid[0], ctx->post_norm[l], h));
      lg.x = h;
    }
    TRY(run_linear<T>(ctx, lg));
    Lin ld{};
    ld.M = M; ld.N = H; ld.K = I; ld.W = ctx->down_w[l]; ld.x = act; ld.epi = EPI_F32; ld.out = d_d; ld.ldo = H;
    ld.ksplit_ok = 1; ld.ksplit_used = &n_dd; ld.split_stride = res_stride; ld.kind = KK_DOWN;
    TRY(run_linear<T>(ctx, ld));
  }
  // ---- final norm + LM head on the sampled rows
  Lin lh{};
  lh.N = c.vocab; lh.K = H; lh.W = c_lm_head_of(ctx); lh.epi = EPI_F32; lh.out = ctx->logits; lh.ldo = c.vocab;
  lh.kind = KK_LM_HEAD;
  if (logit_rows == nullptr && fuse_norm) {
    lh.M = M; lh.norm = 1; lh.r_in = resid[0]; lh.delta = d_d; lh.n_delta = n_dd; lh.delta_stride = res_stride;
    lh.gain = c_final_norm_of(ctx); lh.eps = c.rms_eps;
  } else {
    const int rows = logit_rows ? n_logits : M;
    TRY(run_norm<T>(ctx, rows, resid[0], d_d, n_dd, res_stride, nullptr, nullptr, logit_rows, nullptr,
                    c_final_norm_of(ctx), h));
    lh.M = rows; lh.x = h;
  }
  lh.smp = smp;
  lh.sampled = sampled;
  TRY(run_linear<T>(ctx, lh));
  return STEP_OK;
}

}  // namespace


namespace {

// Mixed-step metadata: rng[2] | tok | pos | slot | row_req | row_len [TM] | qsl [RM+1] | req_len [RM]
// | bt [RM*W] | logit_idx [LM] | temp [LM] | tile_req [tiles] | tile_q0 [tiles] | dec_rows [RM] | n_logits
struct MixedMeta {
  uint64_t* rng;
  int *tok, *pos, *slot, *row_req, *row_len, *qsl, *req_len, *bt, *lidx;
  float* temp;
  int *tile_req, *tile_q0;
  int* dec_rows;   // packed rows of the decode requests, -1 past them (bucketed plan)
  int* n_logits;   // sampled rows (bucketed plan)
  int* topk;       // [LM] per sampled row
  float* topp;
};
MixedMeta mixed_meta(char* base, const Layout& L, int W) {
  MixedMeta m;
  const int TM = L.TM, RM = L.RM, LM = L.LM;
  const int tiles = TM / 16 + RM + 1;
  m.rng = reinterpret_cast<uint64_t*>(base);
  m.tok = reinterpret_cast<int*>(base + 16);
  m.pos = m.tok + TM;
  m.slot = m.pos + TM;
  m.row_req = m.slot + TM;
  m.row_len = m.row_req + TM;
  m.qsl = m.row_len + TM;
  m.req_len = m.qsl + RM + 1;
  m.bt = m.req_len + RM;
  m.lidx = m.bt + static_cast<size_t>(RM) * W;
  m.temp = reinterpret_cast<float*>(m.lidx + LM);
  m.tile_req = reinterpret_cast<int*>(m.temp + LM);
  m.tile_q0 = m.tile_req + tiles;
  m.dec_rows = m.tile_q0 + tiles;
  m.n_logits = m.dec_rows + RM;
  m.topk = m.n_logits + 1;
  m.topp = reinterpret_cast<float*>(m.topk + LM);
  return m;
}

// The single-row decode step as one persistent kernel (see persistent.h), instantiated for the
// widths validate_config admits: hidden 1024 (2 vectors per lane), 2048 query dims (4),
// intermediate 3072 (6), 2 query heads per KV head.
template <class T>
int run_persist(step_ctx* ctx, const DecodeMeta& m) {
  if constexpr (std::is_same<T, F32>::value) {
    return fail(ctx, STEP_EUNSUPPORTED, "persistent decode has no fp32 kernel");
  } else {
    const step_config& c = ctx->cfg;
    const Layout& L = ctx->lay;
    char* ws = ctx->ws;
    PersistArgs a{};
    a.layers = c.layers; a.nq = c.q_heads; a.nkv = c.kv_heads; a.vocab = c.vocab; a.max_position = c.max_position;
    a.eps = c.rms_eps; a.scale = 1.0f / std::sqrt(static_cast<float>(c.head_dim));
    a.lw = reinterpret_cast<const PLayer*>(ws + L.p_lw);
    a.embed = c_embed_of(ctx); a.lm_head = c_lm_head_of(ctx); a.final_norm = c_final_norm_of(ctx);
    a.ids = m.ids; a.pos = m.pos; a.slot = m.slot; a.len = m.len; a.bt = m.bt;
    a.bt_stride = c.max_blocks_per_seq; a.num_blocks = c.num_blocks; a.splits_alloc = L.p_splits;
    a.rope_cos = reinterpret_cast<const float*>(ws + L.rope_cos);
    a.rope_sin = reinterpret_cast<const float*>(ws + L.rope_sin);
    a.x_qkv = reinterpret_cast<uint64_t*>(ws + L.p_qkv);
    a.x_part = reinterpret_cast<uint64_t*>(ws + L.p_part);
    a.x_attn = reinterpret_cast<uint64_t*>(ws + L.p_attn);
    a.x_o = reinterpret_cast<uint64_t*>(ws + L.p_o);
    a.x_act = reinterpret_cast<uint64_t*>(ws + L.p_act);
    a.x_down = reinterpret_cast<uint64_t*>(ws + L.p_down);
    unsigned* ctl = reinterpret_cast<unsigned*>(ws + L.p_ctl);
    a.epoch = ctl; a.done = ctl + 1; a.err = reinterpret_cast<int*>(ctl + 2);
    a.stamps = ctx->p_stamp_next ? reinterpret_cast<unsigned long long*>(ws + L.p_stamps) : nullptr;
    a.logits = ctx->logits;
    // without top-k / top-p filters the sampler runs inside the kernel, after the LM head
    a.sample = c.sampling_filters ? 0 : 1;
    a.temp = m.temp; a.rng = m.rng; a.tokens = ctx->tokens; a.history = ctx->history;
    a.cand = reinterpret_cast<uint64_t*>(ws + L.p_cand);
    pre_launch(ctx, KK_PERSIST);
    if (persist_tpw(c) == 1) launch((k_persist_decode<T, 2, 4, 6, 2, 1>), dim3(ctx->p_nb), dim3(gr::kPThreads), 0, ctx->stream, a);
    else launch((k_persist_decode<T, 2, 4, 6, 2, 2>), dim3(ctx->p_nb), dim3(gr::kPThreads), 0, ctx->stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(ctx, STEP_EHIP, "persistent decode launch failed: %s", hipGetErrorString(e));
    return STEP_OK;
  }
}

template <class T>
int run_decode(step_ctx* ctx, int B) {
  const step_config& c = ctx->cfg;
  const Layout& L = ctx->lay;
  const int W = c.max_blocks_per_seq;
  DecodeMeta m = decode_meta(ctx->ws + L.dmeta, c.max_batch, W);
  if (ctx->p_nb > 0 && B == 1) {
    TRY(run_persist<T>(ctx, m));
    if (!c.sampling_filters) return STEP_OK;
    // the persistent kernel's give-up word stops the separate sampler's token and advance too
    return run_sample(ctx, ctx->logits, B, c.vocab, c.vocab, m.temp, nullptr, m.rng, 0, 0, ctx->tokens, 1, m.ids, m.pos,
                      m.len, m.slot, m.bt, W, ctx->history, c.max_position, nullptr, m.topk, m.topp,
                      reinterpret_cast<const int*>(ctx->ws + L.p_ctl) + 2);
  }
  const float* q = reinterpret_cast<const float*>(ctx->ws + L.q);
  void* attn_o = ctx->ws + L.attn_o;
  (void)q;
  auto attn = [&](int l, int n_qkv) {
    return run_attn_rows<T>(ctx, l, B, nullptr, n_qkv, m.pos, m.slot, m.bt, W, nullptr, m.len, c.max_position, attn_o);
  };
  // without filters the sampler may run in the LM head's epilogue (streaming GEMV rows)
  const SampleArgs smp = sample_args(ctx, ctx->logits, c.vocab, c.vocab, m.temp, nullptr, m.rng, 0, 0, ctx->tokens, 1,
                                     m.ids, m.pos, m.len, m.slot, m.bt, W, ctx->history, c.max_position, nullptr,
                                     nullptr);
  bool sampled = false;
  TRY(run_layers<T>(ctx, B, m.ids, m.pos, m.slot, 0, nullptr, true, attn, c.sampling_filters ? nullptr : &smp,
                    &sampled));
  if (sampled) return STEP_OK;
  return run_sample(ctx, ctx->logits, B, c.vocab, c.vocab, m.temp, nullptr, m.rng, 0, 0, ctx->tokens, 1, m.ids, m.pos,
                    m.len, m.slot, m.bt, W, ctx->history, c.max_position, nullptr,
                    c.sampling_filters ? m.topk : nullptr, c.sampling_filters ? m.topp : nullptr);
}

int run_decode_any(step_ctx* ctx, int B) {
  switch (ctx->cfg.dtype) {
    case STEP_F32: return run_decode<F32>(ctx, B);
    case STEP_BF16: return run_decode<BF16>(ctx, B);
    default: return run_decode<F16>(ctx, B);
  }
}

struct MixedPlan {
  int T, n_pre_tok, n_pre_req, n_dec, n_logits, max_len, mode, n_tiles;
  bool fixed = false;   // bucketed plan: every launch shape depends on T (the bucket) only
};

// The launch plan of a mixed step padded to token-count bucket TB: TB token rows, a tile list of
// TB/16 + max_reqs entries, decode-row attention over min(max_reqs, TM) listed rows with splits
// sized for max_position, and max_logit_rows logits rows; the real counts live in the metadata.
MixedPlan fixed_plan(const step_ctx* ctx, int TB) {
  MixedPlan p{};
  p.T = TB;
  p.n_logits = ctx->lay.LM;
  p.max_len = ctx->cfg.max_position;
  p.mode = 0;
  p.n_tiles = TB / 16 + ctx->lay.RM;
  p.fixed = true;
  return p;
}

template <class T>
int run_attn_prefill(step_ctx* ctx, int layer, const MixedPlan& p, const MixedMeta& m, const float* q, void* out) {
  const step_config& c = ctx->cfg;
  PrefillArgs a{};
  a.nq = c.q_heads; a.nkv = c.kv_heads; a.q = q;
  a.k_pool = ctx->k_pool[layer]; a.v_pool = ctx->v_pool[layer];
  a.block_table = m.bt; a.bt_stride = c.max_blocks_per_seq;
  a.tile_req = m.tile_req; a.tile_q0 = m.tile_q0; a.qsl = m.qsl; a.pos = m.pos;
  a.num_blocks = c.num_blocks;
  a.scale = 1.0f / sqrtf(static_cast<float>(c.head_dim));
  a.out = out;
  dim3 grid(p.n_tiles, c.q_heads);
  pre_launch(ctx, KK_PREFILL_ATTN);
  if (c.head_dim == 64) launch((k_attn_prefill<T, 64>), grid, dim3(256), 0, ctx->stream, a);
  else launch((k_attn_prefill<T, 128>), grid, dim3(256), 0, ctx->stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ctx, STEP_EHIP, "prefill attention launch failed: %s", hipGetErrorString(e));
  return STEP_OK;
}

// The two attention launches of a mixed step as parallel branches: rows() on the side stream,
// prefill() on the step's stream, both after the work already enqueued and before what follows
// (inside a capture, two branches of the graph). The join is enqueued even when a launch fails, so
// a capture never ends with an unjoined stream.
template <class Pre, class Rows>
int attn_branches(step_ctx* ctx, Pre&& prefill, Rows&& rows) {
  hipStream_t main = ctx->stream;
  hipError_t e = hipEventRecord(ctx->fork_ev, main);
  if (e == hipSuccess) e = hipStreamWaitEvent(ctx->side_stream, ctx->fork_ev, 0);
  if (e != hipSuccess) return fail(ctx, STEP_EHIP, "attention fork: %s", hipGetErrorString(e));
  ctx->stream = ctx->side_stream;
  const int rc_rows = rows();
  ctx->stream = main;
  const int rc_pre = prefill();
  e = hipEventRecord(ctx->join_ev, ctx->side_stream);
  if (e == hipSuccess) e = hipStreamWaitEvent(main, ctx->join_ev, 0);
  if (e != hipSuccess) return fail(ctx, STEP_EHIP, "attention join: %s", hipGetErrorString(e));
  return rc_rows != STEP_OK ? rc_rows : rc_pre;
}

template <class T>
int run_mixed(step_ctx* ctx, const MixedPlan& p) {
  const step_config& c = ctx->cfg;
  const Layout& L = ctx->lay;
  const int W = c.max_blocks_per_seq;
  MixedMeta m = mixed_meta(ctx->ws + L.mmeta, L, W);
  const float* q = reinterpret_cast<const float*>(ctx->ws + L.q);
  void* attn_o = ctx->ws + L.attn_o;
  const size_t row_elems = static_cast<size_t>(c.q_heads) * c.head_dim;
  auto attn = [&](int l, int) -> int {
    if (p.fixed) {
      if constexpr (std::is_same<T, F32>::value) {
        return run_attn_rows<T>(ctx, l, p.T, q, 0, nullptr, nullptr, m.bt, W, m.row_req, m.row_len, p.max_len, attn_o);
      } else {
        // listed tiles on the packed kernel, listed decode rows on the row kernel (disjoint outputs,
        // side by side: two branches of the bucket's graph)
        return attn_branches(
            ctx, [&] { return run_attn_prefill<T>(ctx, l, p, m, q, attn_o); },
            [&] {
              return run_attn_rows<T>(ctx, l, std::min(L.RM, L.TM), q, 0, nullptr, nullptr, m.bt, W, m.row_req,
                                      m.row_len, p.max_len, attn_o, m.dec_rows);
            });
      }
    }
    if (p.mode == 1 || p.n_pre_tok == 0 || std::is_same<T, F32>::value) {
      // one query row per token: prefill rows see keys [0, pos], decode rows their request's keys
      return run_attn_rows<T>(ctx, l, p.T, q, 0, nullptr, nullptr, m.bt, W, m.row_req, m.row_len, p.max_len, attn_o);
    }
    if constexpr (!std::is_same<T, F32>::value) {
      // chunk tokens packed on MFMA, decode rows one query row each, into disjoint output rows (in
      // turn: launched eagerly, the cross-stream waits cost more than the overlap saves)
      TRY(run_attn_prefill<T>(ctx, l, p, m, q, attn_o));
      if (p.T > p.n_pre_tok) {
        const int off = p.n_pre_tok;
        return run_attn_rows<T>(ctx, l, p.T - off, q + off * row_elems, 0, nullptr, nullptr, m.bt, W, m.row_req + off,
                                m.row_len + off, p.max_len, static_cast<typename T::S*>(attn_o) + off * row_elems);
      }
    }
    return STEP_OK;
  };
  const SampleArgs smp = sample_args(ctx, ctx->logits, c.vocab, c.vocab, m.temp, nullptr, m.rng, 0, 0, ctx->tokens, 0,
                                     nullptr, nullptr, nullptr, nullptr, nullptr, W, nullptr, 0,
                                     p.fixed ? m.n_logits : nullptr, nullptr);
  bool sampled = false;
  TRY(run_layers<T>(ctx, p.T, m.tok, m.pos, m.slot, p.n_logits, m.lidx, false, attn,
                    c.sampling_filters ? nullptr : &smp, &sampled));
  if (sampled) return STEP_OK;
  return run_sample(ctx, ctx->logits, p.n_logits, c.vocab, c.vocab, m.temp, nullptr, m.rng, 0, 0, ctx->tokens, 0,
                    nullptr, nullptr, nullptr, nullptr, nullptr, W, nullptr, 0, p.fixed ? m.n_logits : nullptr,
                    c.sampling_filters ? m.topk : nullptr, c.sampling_filters ? m.topp : nullptr);
}

// Metadata of a mixed step padded to TB tokens with no real rows (capture and warm-up state).
void fill_mixed_padding(const step_ctx* ctx, char* base, int TB) {
  const Layout& L = ctx->lay;
  const int W = ctx->cfg.max_blocks_per_seq;
  MixedMeta m = mixed_meta(base, L, W);
  m.rng[0] = 0;
  m.rng[1] = 0;
  for (int i = 0; i < TB; ++i) { m.tok[i] = 0; m.pos[i] = 0; m.slot[i] = -1; m.row_req[i] = 0; m.row_len[i] = 0; }
  for (int j = 0; j <= L.RM; ++j) m.qsl[j] = 0;
  for (int j = 0; j < L.RM; ++j) { m.req_len[j] = 0; m.dec_rows[j] = -1; }
  std::memset(m.bt, 0, sizeof(int) * static_cast<size_t>(L.RM) * W);
  for (int i = 0; i < L.LM; ++i) { m.lidx[i] = 0; m.temp[i] = 0.f; m.topk[i] = 0; m.topp[i] = 1.f; }
  for (int t = 0; t < TB / 16 + L.RM; ++t) { m.tile_req[t] = -1; m.tile_q0[t] = 0; }
  *m.n_logits = 0;
}

int run_mixed_any(step_ctx* ctx, const MixedPlan& p) {
  switch (ctx->cfg.dtype) {
    case STEP_F32: return run_mixed<F32>(ctx, p);
    case STEP_BF16: return run_mixed<BF16>(ctx, p);
    default: return run_mixed<F16>(ctx, p);
  }
}

char* stage_slot(step_ctx* ctx, int* which) {
  const int i = ctx->stage_next;
  ctx->stage_next ^= 1;
  // the previous copy out of this slot has completed
  if (hipEventSynchronize(ctx->stage_ev[i]) != hipSuccess) return nullptr;
  *which = i;
  return ctx->h_stage[i];
}

// all decode rows padding: token 0, position 0, slot -1, length 0, zero table, greedy
void fill_decode_padding(const step_config& c, char* base) {
  DecodeMeta m = decode_meta(base, c.max_batch, c.max_blocks_per_seq);
  m.rng[0] = 0;
  m.rng[1] = 0;
  for (int i = 0; i < c.max_batch; ++i) {
    m.ids[i] = 0; m.pos[i] = 0; m.slot[i] = -1; m.len[i] = 0; m.temp[i] = 0.f; m.topk[i] = 0; m.topp[i] = 1.f;
  }
  std::memset(m.bt, 0, sizeof(int) * static_cast<size_t>(c.max_batch) * c.max_blocks_per_seq);
}

int bucket_of(const step_config& c, int r) {
  for (int i = 0; i < c.num_buckets; ++i)
    if (c.buckets[i] >= r) return c.buckets[i];
  return -1;
}

int bucket_index(const step_config& c, int b) {
  for (int i = 0; i < c.num_buckets; ++i)
    if (c.buckets[i] == b) return i;
  return -1;
}

}  // namespace

// ================================================================================================
// C ABI

static size_t step_workspace_bytes_body(const step_config* cfg) {
  if (validate_config(nullptr, cfg) != STEP_OK) return 0;
  Layout L{};
  compute_layout(*cfg, L);
  return L.total;
}

static int step_init_body(step_ctx* ctx, const step_config* cfg, const step_weights* w, const step_buffers* b,
                          void* stream, step_ctx** out) {
  auto bail = [&](int rc) {
    // keep the context so the caller can read the message; it is marked dead
    ctx->dead = true;
    *out = ctx;
    return rc;
  };
  int rc = validate_config(ctx, cfg);
  if (rc != STEP_OK) return bail(rc);
  const step_config& c = *cfg;
  ctx->cfg = c;
  if (!w || !b) return bail(fail(ctx, STEP_EINVAL, "weights or buffers is NULL"));
  if (!w->d_embed || !w->d_lm_head || !w->d_final_norm || !w->d_in_norm || !w->d_qkv_w || !w->d_o_w ||
      !w->d_post_norm || !w->d_gate_up_w || !w->d_down_w)
    return bail(fail(ctx, STEP_EINVAL, "a required weight pointer is NULL"));
  if (c.qkv_bias && !w->d_qkv_b) return bail(fail(ctx, STEP_EINVAL, "qkv_bias set but d_qkv_b is NULL"));
  if (c.qk_norm && (!w->d_q_norm || !w->d_k_norm)) return bail(fail(ctx, STEP_EINVAL, "qk_norm set but gains are NULL"));
  ctx->w = *w;
  for (int l = 0; l < c.layers; ++l) {
    ctx->in_norm.push_back(w->d_in_norm[l]);
    ctx->qkv_w.push_back(w->d_qkv_w[l]);
    ctx->qkv_b.push_back(c.qkv_bias ? w->d_qkv_b[l] : nullptr);
    ctx->q_norm.push_back(c.qk_norm ? w->d_q_norm[l] : nullptr);
    ctx->k_norm.push_back(c.qk_norm ? w->d_k_norm[l] : nullptr);
    ctx->o_w.push_back(w->d_o_w[l]);
    ctx->post_norm.push_back(w->d_post_norm[l]);
    ctx->gate_up_w.push_back(w->d_gate_up_w[l]);
    ctx->down_w.push_back(w->d_down_w[l]);
    if (!ctx->in_norm[l] || !ctx->qkv_w[l] || !ctx->o_w[l] || !ctx->post_norm[l] || !ctx->gate_up_w[l] ||
        !ctx->down_w[l] || (c.qkv_bias && !ctx->qkv_b[l]) || (c.qk_norm && (!ctx->q_norm[l] || !ctx->k_norm[l])))
      return bail(fail(ctx, STEP_EINVAL, "NULL weight pointer at layer %d", l));
  }
  if (!b->d_k_pool || !b->d_v_pool || !b->d_logits || !b->d_tokens || !b->d_workspace)
    return bail(fail(ctx, STEP_EINVAL, "a required buffer pointer is NULL"));
  for (int l = 0; l < c.layers; ++l) {
    if (!b->d_k_pool[l] || !b->d_v_pool[l]) return bail(fail(ctx, STEP_EINVAL, "NULL KV pool at layer %d", l));
    ctx->k_pool.push_back(b->d_k_pool[l]);
    ctx->v_pool.push_back(b->d_v_pool[l]);
  }
  compute_layout(c, ctx->lay);
  if (b->workspace_bytes < ctx->lay.total)
    return bail(fail(ctx, STEP_EINVAL, "workspace has %zu bytes, needs %zu", b->workspace_bytes, ctx->lay.total));
  if (reinterpret_cast<uintptr_t>(b->d_workspace) % kAlign)
    return bail(fail(ctx, STEP_EINVAL, "workspace must be 256-byte aligned"));
  ctx->ws = static_cast<char*>(b->d_workspace);
  ctx->logits = b->d_logits;
  ctx->tokens = b->d_tokens;
  ctx->history = b->d_history;
  ctx->stream = static_cast<hipStream_t>(stream);

  auto hip_fail = [&](hipError_t e, const char* what) {
    return bail(fail(ctx, STEP_EHIP, "%s failed: %s", what, hipGetErrorString(e)));
  };
  hipError_t e;
  if ((e = hipStreamCreateWithFlags(&ctx->cap_stream, hipStreamNonBlocking)) != hipSuccess) return hip_fail(e, "hipStreamCreate");
  if ((e = hipStreamCreateWithFlags(&ctx->side_stream, hipStreamNonBlocking)) != hipSuccess) return hip_fail(e, "hipStreamCreate");
  if ((e = hipEventCreateWithFlags(&ctx->fork_ev, hipEventDisableTiming)) != hipSuccess) return hip_fail(e, "hipEventCreate");
  if ((e = hipEventCreateWithFlags(&ctx->join_ev, hipEventDisableTiming)) != hipSuccess) return hip_fail(e, "hipEventCreate");
  ctx->stage_bytes = std::max(ctx->lay.dmeta_bytes, ctx->lay.mmeta_bytes);
  ctx->stage_bytes = std::max(ctx->stage_bytes, 3 * sizeof(float) * static_cast<size_t>(ctx->lay.LM));
  for (int i = 0; i < 2; ++i) {
    if ((e = hipHostMalloc(reinterpret_cast<void**>(&ctx->h_stage[i]), ctx->stage_bytes, hipHostMallocDefault)) != hipSuccess)
      return hip_fail(e, "hipHostMalloc");
    if ((e = hipEventCreateWithFlags(&ctx->stage_ev[i], hipEventDisableTiming)) != hipSuccess) return hip_fail(e, "hipEventCreate");
  }
  // Everything below runs on the private stream, then the caller's stream waits for it.
  hipStream_t s = ctx->cap_stream;
  if ((e = hipMemsetAsync(ctx->ws, 0, ctx->lay.total, s)) != hipSuccess) return hip_fail(e, "hipMemsetAsync(workspace)");
  // RoPE table: angle = pos * theta^(-2i/d) in fp64, cos/sin rounded to fp32
  {
    const int half = c.head_dim / 2;
    std::vector<float> cs(static_cast<size_t>(c.max_position) * half), sn(cs.size());
    for (int p = 0; p < c.max_position; ++p)
      for (int i = 0; i < half; ++i) {
        const double inv = std::pow(static_cast<double>(c.rope_theta), -2.0 * i / c.head_dim);
        const double ang = static_cast<double>(p) * inv;
        cs[static_cast<size_t>(p) * half + i] = static_cast<float>(std::cos(ang));
        sn[static_cast<size_t>(p) * half + i] = static_cast<float>(std::sin(ang));
      }
    if ((e = hipMemcpy(ctx->ws + ctx->lay.rope_cos, cs.data(), sizeof(float) * cs.size(), hipMemcpyHostToDevice)) != hipSuccess)
      return hip_fail(e, "hipMemcpy(rope)");
    if ((e = hipMemcpy(ctx->ws + ctx->lay.rope_sin, sn.data(), sizeof(float) * sn.size(), hipMemcpyHostToDevice)) != hipSuccess)
      return hip_fail(e, "hipMemcpy(rope)");
  }
  // zero the scratch block of every pool
  const size_t blk_bytes = static_cast<size_t>(c.kv_heads) * 16 * c.head_dim * elem_bytes(c.dtype);
  for (int l = 0; l < c.layers; ++l) {
    if ((e = hipMemsetAsync(static_cast<char*>(ctx->k_pool[l]) + blk_bytes * (c.num_blocks - 1), 0, blk_bytes, s)) != hipSuccess)
      return hip_fail(e, "hipMemsetAsync(scratch)");
    if ((e = hipMemsetAsync(static_cast<char*>(ctx->v_pool[l]) + blk_bytes * (c.num_blocks - 1), 0, blk_bytes, s)) != hipSuccess)
      return hip_fail(e, "hipMemsetAsync(scratch)");
  }
  if (c.persistent_decode) {
    // per-layer pointers for the persistent step, and its launch width: one block per CU of the
    // 256 its tiling is built for (each of a block's four compute waves then owns one register tile
    // of every projection, and each of the eight waves at least one LM-head row)
    std::vector<PLayer> pl(c.layers);
    for (int l = 0; l < c.layers; ++l)
      pl[l] = PLayer{ctx->in_norm[l], ctx->qkv_w[l], ctx->qkv_b[l], ctx->q_norm[l], ctx->k_norm[l], ctx->o_w[l],
                     ctx->post_norm[l], ctx->gate_up_w[l], ctx->down_w[l], ctx->k_pool[l], ctx->v_pool[l]};
    if ((e = hipMemcpy(ctx->ws + ctx->lay.p_lw, pl.data(), sizeof(PLayer) * pl.size(), hipMemcpyHostToDevice)) != hipSuccess)
      return hip_fail(e, "hipMemcpy(layer pointers)");
    int dev = 0, cus = 0, per_cu = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return hip_fail(e, "hipGetDevice");
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
      return hip_fail(e, "hipDeviceGetAttribute");
    const bool two = persist_tpw(c) == 2;
    const void* kfn = c.dtype == STEP_BF16
                          ? (two ? reinterpret_cast<const void*>(&k_persist_decode<BF16, 2, 4, 6, 2, 2>)
                                 : reinterpret_cast<const void*>(&k_persist_decode<BF16, 2, 4, 6, 2, 1>))
                          : (two ? reinterpret_cast<const void*>(&k_persist_decode<F16, 2, 4, 6, 2, 2>)
                                 : reinterpret_cast<const void*>(&k_persist_decode<F16, 2, 4, 6, 2, 1>));
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kfn, gr::kPThreads, 0)) != hipSuccess)
      return hip_fail(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
    if (per_cu < 1) return bail(fail(ctx, STEP_EUNSUPPORTED, "persistent decode kernel does not fit on a CU"));
    if (cus < gr::kPBlocks)
      return bail(fail(ctx, STEP_EUNSUPPORTED, "persistent decode needs %d CUs (one block each), the device has %d",
                       gr::kPBlocks, cus));
    ctx->p_nb = gr::kPBlocks;
  }
  fill_decode_padding(c, ctx->h_stage[0]);
  if ((e = hipMemcpyAsync(ctx->ws + ctx->lay.dmeta, ctx->h_stage[0], ctx->lay.dmeta_bytes, hipMemcpyHostToDevice, s)) != hipSuccess)
    return hip_fail(e, "hipMemcpyAsync(meta)");
  if ((e = hipStreamSynchronize(s)) != hipSuccess) return hip_fail(e, "hipStreamSynchronize");

  ctx->graphs.assign(c.num_buckets, nullptr);
  ctx->execs.assign(c.num_buckets, nullptr);
  ctx->kernels_per_bucket.assign(c.num_buckets, 0);
  hipStream_t user = ctx->stream;
  ctx->stream = s;
  for (int bi = c.num_buckets - 1; bi >= 0; --bi) {   // largest bucket first
    const int B = c.buckets[bi];
    // two warm-up steps over all-padding rows: only the scratch block is written
    for (int wup = 0; wup < 2; ++wup) {
      ctx->launches = 0;
      rc = run_decode_any(ctx, B);
      if (rc != STEP_OK) { ctx->stream = user; return bail(rc); }
    }
    ctx->kernels_per_bucket[bi] = ctx->launches;
    if (!c.use_graphs) continue;
    if ((e = hipStreamSynchronize(s)) != hipSuccess) { ctx->stream = user; return hip_fail(e, "hipStreamSynchronize"); }
    if ((e = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal)) != hipSuccess) {
      ctx->stream = user;
      return bail(fail(ctx, STEP_ECAPTURE, "hipStreamBeginCapture: %s", hipGetErrorString(e)));
    }
    ctx->launches = 0;
    rc = run_decode_any(ctx, B);
    hipGraph_t g = nullptr;
    hipError_t ee = hipStreamEndCapture(s, &g);
    if (rc != STEP_OK || ee != hipSuccess || !g) {
      ctx->stream = user;
      if (g) (void)hipGraphDestroy(g);
      return bail(rc != STEP_OK ? rc : fail(ctx, STEP_ECAPTURE, "hipStreamEndCapture: %s", hipGetErrorString(ee)));
    }
    hipGraphExec_t x = nullptr;
    if ((e = hipGraphInstantiate(&x, g, nullptr, nullptr, 0)) != hipSuccess) {
      ctx->stream = user;
      (void)hipGraphDestroy(g);
      return bail(fail(ctx, STEP_ECAPTURE, "hipGraphInstantiate: %s", hipGetErrorString(e)));
    }
    ctx->graphs[bi] = g;
    ctx->execs[bi] = x;
  }
  // mixed-step buckets: all-padding metadata, two warm-ups, then capture (largest first)
  ctx->mgraphs.assign(c.num_mixed_buckets, nullptr);
  ctx->mexecs.assign(c.num_mixed_buckets, nullptr);
  ctx->kernels_per_mbucket.assign(c.num_mixed_buckets, 0);
  for (int bi = c.num_mixed_buckets - 1; bi >= 0; --bi) {
    const int TB = c.mixed_buckets[bi];
    fill_mixed_padding(ctx, ctx->h_stage[0], TB);
    if ((e = hipMemcpyAsync(ctx->ws + ctx->lay.mmeta, ctx->h_stage[0], ctx->lay.mmeta_bytes, hipMemcpyHostToDevice, s)) !=
        hipSuccess) {
      ctx->stream = user;
      return hip_fail(e, "hipMemcpyAsync(mixed meta)");
    }
    if ((e = hipStreamSynchronize(s)) != hipSuccess) { ctx->stream = user; return hip_fail(e, "hipStreamSynchronize"); }
    const MixedPlan mp = fixed_plan(ctx, TB);
    for (int wup = 0; wup < 2; ++wup) {
      ctx->launches = 0;
      rc = run_mixed_any(ctx, mp);
      if (rc != STEP_OK) { ctx->stream = user; return bail(rc); }
    }
    ctx->kernels_per_mbucket[bi] = ctx->launches;
    if (!c.use_graphs) continue;
    if ((e = hipStreamSynchronize(s)) != hipSuccess) { ctx->stream = user; return hip_fail(e, "hipStreamSynchronize"); }
    if ((e = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal)) != hipSuccess) {
      ctx->stream = user;
      return bail(fail(ctx, STEP_ECAPTURE, "hipStreamBeginCapture: %s", hipGetErrorString(e)));
    }
    ctx->launches = 0;
    rc = run_mixed_any(ctx, mp);
    hipGraph_t g = nullptr;
    hipError_t ee = hipStreamEndCapture(s, &g);
    if (rc != STEP_OK || ee != hipSuccess || !g) {
      ctx->stream = user;
      if (g) (void)hipGraphDestroy(g);
      return bail(rc != STEP_OK ? rc : fail(ctx, STEP_ECAPTURE, "hipStreamEndCapture: %s", hipGetErrorString(ee)));
    }
    hipGraphExec_t x = nullptr;
    if ((e = hipGraphInstantiate(&x, g, nullptr, nullptr, 0)) != hipSuccess) {
      ctx->stream = user;
      (void)hipGraphDestroy(g);
      return bail(fail(ctx, STEP_ECAPTURE, "hipGraphInstantiate: %s", hipGetErrorString(e)));
    }
    ctx->mgraphs[bi] = g;
    ctx->mexecs[bi] = x;
  }
  ctx->stream = user;
  // warm-ups moved the Philox step counter: put the padding state back
  fill_decode_padding(c, ctx->h_stage[0]);
  if ((e = hipMemcpyAsync(ctx->ws + ctx->lay.dmeta, ctx->h_stage[0], ctx->lay.dmeta_bytes, hipMemcpyHostToDevice, s)) != hipSuccess)
    return hip_fail(e, "hipMemcpyAsync(meta)");
  if ((e = hipStreamSynchronize(s)) != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  *out = ctx;
  return STEP_OK;
}

static int step_decode_body(step_ctx* ctx, const step_batch* hb) {
  if (!ctx || ctx->dead) return STEP_ESTATE;
  const step_config& c = ctx->cfg;
  int B;
  if (hb) {
    const int r = hb->num_rows;
    if (r < 1 || r > c.max_batch) return fail(ctx, STEP_EINVAL, "num_rows %d outside [1, %d]", r, c.max_batch);
    if (hb->bt_width < 0 || hb->bt_width > c.max_blocks_per_seq)
      return fail(ctx, STEP_EINVAL, "bt_width %d above max_blocks_per_seq %d", hb->bt_width, c.max_blocks_per_seq);
    if (!hb->h_tokens || !hb->h_positions || !hb->h_seq_lens || !hb->h_slot_mapping || (hb->bt_width && !hb->h_block_table))
      return fail(ctx, STEP_EINVAL, "NULL batch array");
    if ((hb->h_top_k || hb->h_top_p) && !c.sampling_filters)
      return fail(ctx, STEP_EINVAL, "top-k / top-p given to a context built without sampling_filters");
    B = bucket_of(c, r);
    if (B < 0) return fail(ctx, STEP_EINVAL, "no bucket holds %d rows", r);
    const int W = c.max_blocks_per_seq;
    const int max_slot = (c.num_blocks - 1) * 16;   // slots of the scratch block are not addressable
    for (int i = 0; i < r; ++i) {
      const int t = hb->h_tokens[i], p = hb->h_positions[i], len = hb->h_seq_lens[i], sl = hb->h_slot_mapping[i];
      if (t < 0 || t >= c.vocab) return fail(ctx, STEP_EINVAL, "row %d: token %d outside the vocabulary", i, t);
      if (p < 0 || p >= c.max_position) return fail(ctx, STEP_EINVAL, "row %d: position %d outside [0, max_position)", i, p);
      if (len < 0 || len > c.max_position || (len + 15) / 16 > hb->bt_width)
        return fail(ctx, STEP_EINVAL, "row %d: seq_len %d needs more blocks than the table holds", i, len);
      if (sl < -1 || sl >= max_slot) return fail(ctx, STEP_EINVAL, "row %d: slot %d outside the pool", i, sl);
      for (int j = 0; j < hb->bt_width; ++j) {
        const int blk = hb->h_block_table[static_cast<size_t>(i) * hb->bt_width + j];
        if (blk < -1 || blk >= c.num_blocks - 1) return fail(ctx, STEP_EINVAL, "row %d: block id %d outside the pool", i, blk);
        if (blk < 0 && j < (len + 15) / 16) return fail(ctx, STEP_EINVAL, "row %d: missing block %d of its keys", i, j);
      }
      // a decode row's new token is its last key, stored at the slot its block table gives
      if (len > 0) {
        if (len != p + 1) return fail(ctx, STEP_EINVAL, "row %d: seq_len %d must be position + 1 = %d", i, len, p + 1);
        const int want = hb->h_block_table[static_cast<size_t>(i) * hb->bt_width + p / 16] * 16 + p % 16;
        if (sl != want) return fail(ctx, STEP_EINVAL, "row %d: slot %d is not the table's slot %d", i, sl, want);
      }
    }
    int slot_i;
    char* st = stage_slot(ctx, &slot_i);
    if (!st) return fail(ctx, STEP_EHIP, "waiting for the staging buffer failed");
    fill_decode_padding(c, st);
    DecodeMeta m = decode_meta(st, c.max_batch, W);
    m.rng[0] = hb->seed;
    m.rng[1] = ctx->step_count;
    for (int i = 0; i < r; ++i) {
      m.ids[i] = hb->h_tokens[i];
      m.pos[i] = hb->h_positions[i];
      m.slot[i] = hb->h_slot_mapping[i];
      m.len[i] = hb->h_seq_lens[i];
      m.temp[i] = hb->h_temperature ? hb->h_temperature[i] : 0.f;
      m.topk[i] = hb->h_top_k ? hb->h_top_k[i] : 0;
      m.topp[i] = hb->h_top_p ? hb->h_top_p[i] : 1.f;
      int* row = m.bt + static_cast<size_t>(i) * W;
      for (int j = 0; j < W; ++j) row[j] = j < hb->bt_width ? hb->h_block_table[static_cast<size_t>(i) * hb->bt_width + j] : -1;
    }
    HIPCHK(ctx, hipMemcpyAsync(ctx->ws + ctx->lay.dmeta, st, ctx->lay.dmeta_bytes, hipMemcpyHostToDevice, ctx->stream));
    HIPCHK(ctx, hipEventRecord(ctx->stage_ev[slot_i], ctx->stream));
    ctx->last_bucket = B;
    ctx->have_batch = true;
  } else {
    if (!ctx->have_batch) return fail(ctx, STEP_EINVAL, "continue step before any batch");
    B = ctx->last_bucket;
  }
  const int bi = bucket_index(c, B);
  if (ctx->execs[bi]) {
    HIPCHK(ctx, hipGraphLaunch(ctx->execs[bi], ctx->stream));
  } else {
    ctx->launches = 0;
    int rc = run_decode_any(ctx, B);
    if (rc != STEP_OK) return rc;
  }
  ctx->step_count++;
  return STEP_OK;
}

static int step_mixed_body(step_ctx* ctx, const step_packed* hp) {
  if (!ctx || ctx->dead) return STEP_ESTATE;
  const step_config& c = ctx->cfg;
  if (!hp) return fail(ctx, STEP_EINVAL, "batch is NULL");
  if (c.max_tokens <= 0) return fail(ctx, STEP_EINVAL, "context built without mixed-step buffers (max_tokens 0)");
  const int T = hp->num_tokens, Rp = hp->num_prefill_reqs, Rd = hp->num_decode_reqs, R = Rp + Rd, NL = hp->num_logits;
  const int W = c.max_blocks_per_seq;
  if (T < 1 || T > c.max_tokens) return fail(ctx, STEP_EINVAL, "num_tokens %d outside [1, %d]", T, c.max_tokens);
  if (Rp < 0 || Rd < 0 || R < 1 || R > c.max_reqs) return fail(ctx, STEP_EINVAL, "request count %d outside [1, %d]", R, c.max_reqs);
  if (NL < 1 || NL > c.max_logit_rows) return fail(ctx, STEP_EINVAL, "num_logits %d outside [1, %d]", NL, c.max_logit_rows);
  if (hp->bt_width < 1 || hp->bt_width > W) return fail(ctx, STEP_EINVAL, "bt_width %d outside [1, %d]", hp->bt_width, W);
  if (!hp->h_query_start_loc || !hp->h_seq_lens || !hp->h_tokens || !hp->h_positions || !hp->h_slot_mapping ||
      !hp->h_block_table || !hp->h_logits_indices)
    return fail(ctx, STEP_EINVAL, "NULL batch array");
  if (hp->prefill_attention != 0 && hp->prefill_attention != 1)
    return fail(ctx, STEP_EINVAL, "prefill_attention must be 0 or 1");
  if ((hp->h_top_k || hp->h_top_p) && !c.sampling_filters)
    return fail(ctx, STEP_EINVAL, "top-k / top-p given to a context built without sampling_filters");
  const int* qsl = hp->h_query_start_loc;
  if (qsl[0] != 0 || qsl[R] != T) return fail(ctx, STEP_EINVAL, "query_start_loc must run from 0 to num_tokens");
  for (int j = 0; j < R; ++j) {
    if (qsl[j + 1] <= qsl[j]) return fail(ctx, STEP_EINVAL, "request %d has no tokens", j);
    if (j >= Rp && qsl[j + 1] - qsl[j] != 1) return fail(ctx, STEP_EINVAL, "decode request %d must have one token", j);
    const int len = hp->h_seq_lens[j];
    if (len < 1 || len > c.max_position || (len + 15) / 16 > hp->bt_width)
      return fail(ctx, STEP_EINVAL, "request %d: seq_len %d does not fit the block table", j, len);
    for (int b = 0; b < (len + 15) / 16; ++b) {
      const int blk = hp->h_block_table[static_cast<size_t>(j) * hp->bt_width + b];
      if (blk < 0 || blk >= c.num_blocks - 1) return fail(ctx, STEP_EINVAL, "request %d: block id %d outside the pool", j, blk);
    }
  }
  const int max_slot = (c.num_blocks - 1) * 16;
  int max_len = 1;
  for (int j = 0; j < R; ++j)
    for (int i = qsl[j]; i < qsl[j + 1]; ++i) {
      const int t = hp->h_tokens[i], p = hp->h_positions[i], sl = hp->h_slot_mapping[i];
      if (t < 0 || t >= c.vocab) return fail(ctx, STEP_EINVAL, "token row %d: id %d outside the vocabulary", i, t);
      if (p < 0 || p >= hp->h_seq_lens[j]) return fail(ctx, STEP_EINVAL, "token row %d: position %d not below its seq_len", i, p);
      if (sl < -1 || sl >= max_slot) return fail(ctx, STEP_EINVAL, "token row %d: slot %d outside the pool", i, sl);
      max_len = std::max(max_len, p + 1);
    }
  for (int i = 0; i < NL; ++i)
    if (hp->h_logits_indices[i] < 0 || hp->h_logits_indices[i] >= T)
      return fail(ctx, STEP_EINVAL, "logits index %d outside the packed tokens", hp->h_logits_indices[i]);
  // a prefill chunk holds the last positions of its request: pos = seq_len - n + i
  for (int j = 0; j < Rp; ++j) {
    const int n = qsl[j + 1] - qsl[j];
    for (int i = qsl[j]; i < qsl[j + 1]; ++i)
      if (hp->h_positions[i] != hp->h_seq_lens[j] - n + (i - qsl[j]))
        return fail(ctx, STEP_EINVAL, "request %d: chunk positions must be seq_len - %d .. seq_len - 1", j, n);
  }
  // bucketed plan: the smallest mixed bucket that holds the step (packed prefill attention only)
  int mbi = -1;
  if (hp->prefill_attention == 0)
    for (int i = 0; i < c.num_mixed_buckets; ++i)
      if (c.mixed_buckets[i] >= T) { mbi = i; break; }
  int slot_i;
  char* st = stage_slot(ctx, &slot_i);
  if (!st) return fail(ctx, STEP_EHIP, "waiting for the staging buffer failed");
  MixedMeta m = mixed_meta(st, ctx->lay, W);
  if (mbi >= 0) fill_mixed_padding(ctx, st, c.mixed_buckets[mbi]);
  m.rng[0] = hp->seed;
  m.rng[1] = ctx->step_count;
  for (int j = 0; j < R; ++j) {
    for (int i = qsl[j]; i < qsl[j + 1]; ++i) {
      m.tok[i] = hp->h_tokens[i];
      m.pos[i] = hp->h_positions[i];
      m.slot[i] = hp->h_slot_mapping[i];
      m.row_req[i] = j;
      m.row_len[i] = (j < Rp) ? hp->h_positions[i] + 1 : hp->h_seq_lens[j];
    }
    m.req_len[j] = hp->h_seq_lens[j];
    int* row = m.bt + static_cast<size_t>(j) * W;
    for (int b = 0; b < W; ++b) row[b] = b < hp->bt_width ? hp->h_block_table[static_cast<size_t>(j) * hp->bt_width + b] : -1;
  }
  for (int j = 0; j <= R; ++j) m.qsl[j] = qsl[j];
  int n_tiles = 0;
  for (int j = 0; j < Rp; ++j)
    for (int q0 = qsl[j]; q0 < qsl[j + 1]; q0 += 16) {
      m.tile_req[n_tiles] = j;
      m.tile_q0[n_tiles] = q0;
      ++n_tiles;
    }
  for (int i = 0; i < NL; ++i) {
    m.lidx[i] = hp->h_logits_indices[i];
    m.temp[i] = hp->h_temperature ? hp->h_temperature[i] : 0.f;
    m.topk[i] = hp->h_top_k ? hp->h_top_k[i] : 0;
    m.topp[i] = hp->h_top_p ? hp->h_top_p[i] : 1.f;
  }
  for (int j = Rp; j < R; ++j) m.dec_rows[j - Rp] = qsl[j];
  *m.n_logits = NL;
  HIPCHK(ctx, hipMemcpyAsync(ctx->ws + ctx->lay.mmeta, st, ctx->lay.mmeta_bytes, hipMemcpyHostToDevice, ctx->stream));
  HIPCHK(ctx, hipEventRecord(ctx->stage_ev[slot_i], ctx->stream));
  ctx->launches = 0;
  int rc;
  if (mbi >= 0) {
    ctx->last_mixed_bucket = c.mixed_buckets[mbi];
    if (ctx->mexecs[mbi]) {
      HIPCHK(ctx, hipGraphLaunch(ctx->mexecs[mbi], ctx->stream));
      ctx->launches = ctx->kernels_per_mbucket[mbi];
      rc = STEP_OK;
    } else {
      rc = run_mixed_any(ctx, fixed_plan(ctx, c.mixed_buckets[mbi]));
    }
  } else {
    ctx->last_mixed_bucket = 0;
    MixedPlan p{T, qsl[Rp], Rp, Rd, NL, max_len, hp->prefill_attention, n_tiles};
    rc = run_mixed_any(ctx, p);
  }
  if (rc != STEP_OK) return rc;
  ctx->step_count++;
  return STEP_OK;
}

extern "C" int step_last_mixed_bucket(const step_ctx* ctx) { return ctx ? ctx->last_mixed_bucket : STEP_ESTATE; }

static int step_sample_body(step_ctx* ctx, const float* d_logits, int32_t rows, int32_t ld, int32_t vocab,
                           const float* h_temperature, const int32_t* h_top_k, const float* h_top_p,
                           const float* d_uniforms, uint64_t seed, uint64_t counter, int32_t* d_tokens_out) {
  if (!ctx || ctx->dead) return STEP_ESTATE;
  if (!d_logits || !d_tokens_out) return fail(ctx, STEP_EINVAL, "NULL logits or tokens");
  if (rows < 1 || rows > ctx->lay.LM) return fail(ctx, STEP_EINVAL, "rows %d outside [1, %d]", rows, ctx->lay.LM);
  if (vocab < 1 || vocab > ctx->cfg.vocab || ld < vocab) return fail(ctx, STEP_EINVAL, "bad vocab %d / ld %d", vocab, ld);
  float* temp = nullptr;
  int* topk = nullptr;
  float* topp = nullptr;
  if (h_temperature) {
    // temperature | top_k | top_p staged together, one copy
    const size_t LM = static_cast<size_t>(ctx->lay.LM);
    int slot_i;
    char* st = stage_slot(ctx, &slot_i);
    if (!st) return fail(ctx, STEP_EHIP, "waiting for the staging buffer failed");
    float* s_temp = reinterpret_cast<float*>(st);
    int* s_topk = reinterpret_cast<int*>(st + sizeof(float) * LM);
    float* s_topp = reinterpret_cast<float*>(st + 2 * sizeof(float) * LM);
    for (int i = 0; i < rows; ++i) {
      s_temp[i] = h_temperature[i];
      s_topk[i] = h_top_k ? h_top_k[i] : 0;
      s_topp[i] = h_top_p ? h_top_p[i] : 1.f;
    }
    char* dst = ctx->ws + ctx->lay.samp_temp;
    HIPCHK(ctx, hipMemcpyAsync(dst, st, 3 * sizeof(float) * LM, hipMemcpyHostToDevice, ctx->stream));
    HIPCHK(ctx, hipEventRecord(ctx->stage_ev[slot_i], ctx->stream));
    temp = reinterpret_cast<float*>(dst);
    if (h_top_k) topk = reinterpret_cast<int*>(ctx->ws + ctx->lay.samp_topk);
    if (h_top_p) topp = reinterpret_cast<float*>(ctx->ws + ctx->lay.samp_topp);
  }
  return run_sample(ctx, d_logits, rows, ld, vocab, temp, d_uniforms, nullptr, seed, counter, d_tokens_out, 0, nullptr,
                    nullptr, nullptr, nullptr, nullptr, 0, nullptr, 0, nullptr, topk, topp);
}

static int step_profile_decode_body(step_ctx* ctx, int32_t max_kernels, float* h_ms, int32_t* h_kind) {
  if (!ctx || ctx->dead) return STEP_ESTATE;
  if (!ctx->have_batch) return fail(ctx, STEP_EINVAL, "profile step before any batch");
  if (max_kernels < 1 || !h_ms || !h_kind) return fail(ctx, STEP_EINVAL, "bad profile buffers");
  const size_t nev = static_cast<size_t>(max_kernels);
  while (ctx->prof_ev.size() < nev) {
    hipEvent_t e0, e1;
    HIPCHK(ctx, hipEventCreate(&e0));
    ctx->prof_ev.push_back(e0);
    HIPCHK(ctx, hipEventCreate(&e1));
    ctx->prof_ev_end.push_back(e1);
  }
  ctx->prof_kind.assign(ctx->prof_ev.size(), -1);
  hipLaunchKernelGGL(k_hold, dim3(1), dim3(64), 0, ctx->stream, 1000);
  HIPCHK(ctx, hipGetLastError());
  const bool stamps = ctx->p_nb > 0 && ctx->last_bucket == 1;
  if (stamps) {
    HIPCHK(ctx, hipMemsetAsync(ctx->ws + ctx->lay.p_stamps, 0, sizeof(unsigned long long) * gr::kPStamps, ctx->stream));
  }
  ctx->launches = 0;
  ctx->prof_on = true;
  ctx->p_stamp_next = stamps;
  const int rc = run_decode_any(ctx, ctx->last_bucket);
  ctx->prof_on = false;
  ctx->p_stamp_next = false;
  g_prof_next = ProfSlot{};
  if (rc != STEP_OK) return rc;
  if (stamps) {
    ctx->p_stamps.assign(gr::kPStamps, 0ull);
    HIPCHK(ctx, hipMemcpyAsync(ctx->p_stamps.data(), ctx->ws + ctx->lay.p_stamps, sizeof(unsigned long long) * gr::kPStamps,
                               hipMemcpyDeviceToHost, ctx->stream));
  }
  const int n = std::min(ctx->launches, max_kernels);
  HIPCHK(ctx, hipStreamSynchronize(ctx->stream));
  for (int i = 0; i < n; ++i) {
    float ms = 0.f;
    HIPCHK(ctx, hipEventElapsedTime(&ms, ctx->prof_ev[i], ctx->prof_ev_end[i]));
    h_ms[i] = ms;
    h_kind[i] = ctx->prof_kind[i];
  }
  ctx->step_count++;
  return ctx->launches;
}

extern "C" int step_phase_stamps(const step_ctx* ctx, int32_t max_stamps, double* h_us) {
  if (!ctx || ctx->dead) return STEP_ESTATE;
  if (max_stamps < 0 || (max_stamps > 0 && !h_us)) return STEP_EINVAL;
  if (ctx->p_stamps.empty()) return 0;
  const int n = std::min(max_stamps, gr::kPStamps);
  const unsigned long long t0 = ctx->p_stamps[0];
  for (int i = 0; i < n; ++i)
    h_us[i] = ctx->p_stamps[i] ? static_cast<double>(ctx->p_stamps[i] - t0) * 0.01 : -1.0;   // 100 MHz clock
  return gr::kPStamps;
}

static int step_device_status_body(step_ctx* ctx) {
  if (!ctx || ctx->dead) return STEP_ESTATE;
  if (ctx->p_nb == 0) return STEP_OK;
  HIPCHK(ctx, hipStreamSynchronize(ctx->stream));
  int* err = reinterpret_cast<int*>(ctx->ws + ctx->lay.p_ctl) + 2;
  int v = 0;
  HIPCHK(ctx, hipMemcpy(&v, err, sizeof v, hipMemcpyDeviceToHost));
  if (v == 0) return STEP_OK;
  HIPCHK(ctx, hipMemset(err, 0, sizeof v));
  return fail(ctx, STEP_EHIP, "persistent decode step: a wait gave up (site %d); that step's outputs are invalid", v);
}

// ------------------------------------------------------------------------------------------------
// Exported entry points: each runs its body under a catch-all, so no C++ exception (a failed host
// allocation in a std::vector or std::string, say) ever unwinds across the C ABI.

#define STEP_GUARDED(ctx, body)                                                          \
  try {                                                                                  \
    return body;                                                                         \
  } catch (const std::bad_alloc&) {                                                      \
    return fail((ctx), STEP_EHIP, "host memory allocation failed");                      \
  } catch (...) {                                                                        \
    return fail((ctx), STEP_EHIP, "unexpected C++ exception inside the library");        \
  }

extern "C" size_t step_workspace_bytes(const step_config* cfg) {
  try {
    return step_workspace_bytes_body(cfg);
  } catch (...) {
    return 0;
  }
}

extern "C" int step_init(const step_config* cfg, const step_weights* w, const step_buffers* b, void* stream,
                         step_ctx** out) {
  if (!out) return STEP_EINVAL;
  *out = nullptr;
  step_ctx* ctx = new (std::nothrow) step_ctx();
  if (!ctx) return STEP_EHIP;
  try {
    return step_init_body(ctx, cfg, w, b, stream, out);
  } catch (...) {
    // the context is handed back dead so that the caller can read the message and destroy it
    ctx->dead = true;
    *out = ctx;
    return fail(ctx, STEP_EHIP, "host memory allocation failed during step_init");
  }
}

extern "C" int step_decode(step_ctx* ctx, const step_batch* hb) { STEP_GUARDED(ctx, step_decode_body(ctx, hb)) }

extern "C" int step_mixed(step_ctx* ctx, const step_packed* hp) { STEP_GUARDED(ctx, step_mixed_body(ctx, hp)) }

extern "C" int step_sample(step_ctx* ctx, const float* d_logits, int32_t rows, int32_t ld, int32_t vocab,
                           const float* h_temperature, const int32_t* h_top_k, const float* h_top_p,
                           const float* d_uniforms, uint64_t seed, uint64_t counter, int32_t* d_tokens_out) {
  STEP_GUARDED(ctx, step_sample_body(ctx, d_logits, rows, ld, vocab, h_temperature, h_top_k, h_top_p, d_uniforms, seed,
                                     counter, d_tokens_out))
}

extern "C" int step_profile_decode(step_ctx* ctx, int32_t max_kernels, float* h_ms, int32_t* h_kind) {
  STEP_GUARDED(ctx, step_profile_decode_body(ctx, max_kernels, h_ms, h_kind))
}

extern "C" int step_device_status(step_ctx* ctx) { STEP_GUARDED(ctx, step_device_status_body(ctx)) }

extern "C" int step_set_device_status(step_ctx* ctx, int32_t site) {
  if (!ctx || ctx->dead) return STEP_ESTATE;
  if (ctx->p_nb == 0) return fail(ctx, STEP_EINVAL, "the context has no persistent decode step");
  if (site <= 0) return fail(ctx, STEP_EINVAL, "site %d: must be positive", site);
  int* err = reinterpret_cast<int*>(ctx->ws + ctx->lay.p_ctl) + 2;
  HIPCHK(ctx, hipStreamSynchronize(ctx->stream));
  HIPCHK(ctx, hipMemcpy(err, &site, sizeof site, hipMemcpyHostToDevice));
  return STEP_OK;
}

extern "C" int32_t step_attention_slots(const step_config* cfg, int32_t rows, int32_t max_len, int64_t* capacity) {
  try {
    if (validate_config(nullptr, cfg) != STEP_OK) return STEP_EINVAL;
    Layout L{};
    compute_layout(*cfg, L);
    if (capacity) *capacity = static_cast<int64_t>(L.attn_slots);
    if (rows < 1 || rows > L.TM || max_len < 1 || max_len > cfg->max_position) return STEP_EINVAL;
    return static_cast<int32_t>(attn_slot_demand(rows, max_len, *cfg));
  } catch (...) {
    return STEP_EHIP;
  }
}

extern "C" const char* step_kernel_kind_name(int32_t kind) {
  return (kind >= 0 && kind < KK_COUNT) ? kKindNames[kind] : "unknown";
}

extern "C" int step_last_bucket(const step_ctx* ctx) { return ctx ? ctx->last_bucket : STEP_ESTATE; }

extern "C" int step_kernels_per_decode(const step_ctx* ctx, int32_t bucket) {
  if (!ctx || ctx->dead) return STEP_ESTATE;
  const int bi = bucket_index(ctx->cfg, bucket);
  if (bi < 0) return STEP_EINVAL;
  return ctx->kernels_per_bucket[bi];
}

extern "C" const char* step_last_error(const step_ctx* ctx) { return ctx ? ctx->err.c_str() : "NULL context"; }

extern "C" void step_destroy(step_ctx* ctx) {
  if (!ctx) return;
  // teardown is best effort: errors here have no caller left to report to
  if (ctx->cap_stream) (void)hipStreamSynchronize(ctx->cap_stream);
  if (ctx->stream || !ctx->dead) (void)hipStreamSynchronize(ctx->stream);
  for (auto& x : ctx->execs)
    if (x) (void)hipGraphExecDestroy(x);
  for (auto& g : ctx->graphs)
    if (g) (void)hipGraphDestroy(g);
  for (auto& x : ctx->mexecs)
    if (x) (void)hipGraphExecDestroy(x);
  for (auto& g : ctx->mgraphs)
    if (g) (void)hipGraphDestroy(g);
  for (int i = 0; i < 2; ++i) {
    if (ctx->stage_ev[i]) (void)hipEventDestroy(ctx->stage_ev[i]);
    if (ctx->h_stage[i]) (void)hipHostFree(ctx->h_stage[i]);
  }
  if (ctx->cap_stream) (void)hipStreamDestroy(ctx->cap_stream);
  if (ctx->side_stream) (void)hipStreamSynchronize(ctx->side_stream);
  if (ctx->side_stream) (void)hipStreamDestroy(ctx->side_stream);
  if (ctx->fork_ev) (void)hipEventDestroy(ctx->fork_ev);
  if (ctx->join_ev) (void)hipEventDestroy(ctx->join_ev);
  for (auto& e : ctx->prof_ev) (void)hipEventDestroy(e);
  for (auto& e : ctx->prof_ev_end) (void)hipEventDestroy(e);
  delete ctx;
}
