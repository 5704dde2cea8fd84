// QK-norm + RoPE + paged KV write, and attention over the paged KV pool.
//
// Pool layout per layer: K is [num_blocks][kv_heads][block_size = 16][head_dim] (key-major) and V is
// [num_blocks][kv_heads][head_dim][block_size = 16] (dim-major), so one (block, kv head) tile of
// either is contiguous (4 KiB at head_dim 128 in 16-bit types). Key-major K rows are the row
// operand of the score product; dim-major V gives each lane four consecutive keys of one dim in a
// single 8-byte load, the operand layout of the value product.
// A row with slot -1 (padding) writes its K and V to the scratch block num_blocks - 1, which no
// block table holds ("Removing overhead: fusion, graphs and async scheduling", section "CUDA
// graphs for a changing batch"). A row with seq_len 0 gets a zero attention output.
#pragma once
#include "common.h"
#include "gemm.h"

namespace gr {

constexpr int kBlk = 16;  // tokens per KV block

// element offsets in one layer's pools of token `off` of block `blk`, kv head g: K row start, V dim 0
__device__ inline size_t pool_k_at(int blk, int nkv, int g, int off, int d) {
  return ((static_cast<size_t>(blk) * nkv + g) * kBlk + off) * d;
}
__device__ inline size_t pool_v_at(int blk, int nkv, int g, int off, int d) {
  return (static_cast<size_t>(blk) * nkv + g) * kBlk * d + off;   // dim i at + i * kBlk
}

// One wave per (row, head). Heads [0, nq) are query heads: RMSNorm over head_dim (qk_norm), then
// rotate-half RoPE at the row's position, stored fp32 to q_out. Heads [nq, nq + nkv) are KV heads:
// k gets the same treatment with its own gain, v is copied; both go to the pool slot.
template <class T>
__global__ __launch_bounds__(64) void k_qkv_post(int nq, int nkv, int d, const float* __restrict__ qkv,
                                                 int n_parts, size_t part_stride, const int* __restrict__ pos,
                                                 const int* __restrict__ slot, const float* __restrict__ rope_cos,
                                                 const float* __restrict__ rope_sin, const void* __restrict__ q_norm,
                                                 const void* __restrict__ k_norm, float eps, float* __restrict__ q_out,
                                                 void* __restrict__ k_pool, void* __restrict__ v_pool, int num_blocks) {
  using S = typename T::S;
  const int row = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const int half = d / 2;
  const int ld = (nq + 2 * nkv) * d;
  const bool is_q = h < nq;
  const int g = h - nq;
  const int col = is_q ? h * d : (nq + g) * d;
  const bool act = lane < half;
  // every load first (the first four partials of each element at once), then the arithmetic; the
  // partials are summed in order
  constexpr int NP = 4;
  const float* base = qkv + static_cast<size_t>(row) * ld;
  auto issue = [&](float(&dst)[NP], int c) {
#pragma unroll
    for (int k = 0; k < NP; ++k) dst[k] = (act && k < n_parts) ? base[k * part_stride + c] : 0.f;
  };
  auto sum = [&](const float(&src)[NP], int c) -> float {
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < NP; ++k)
      if (k < n_parts) v += src[k];
    for (int k = NP; k < n_parts; ++k) v += base[k * part_stride + c];
    return v;
  };
  float p0[NP], p1[NP], pv0[NP], pv1[NP];
  const int vcol = (nq + nkv + g) * d;
  issue(p0, col + lane);
  issue(p1, col + lane + half);
  if (!is_q) {
    issue(pv0, vcol + lane);
    issue(pv1, vcol + lane + half);
  }
  const void* gain = is_q ? q_norm : k_norm;
  const S* gw = static_cast<const S*>(gain);
  const float g0 = (gain && act) ? T::to_f(gw[lane]) : 0.f, g1 = (gain && act) ? T::to_f(gw[lane + half]) : 0.f;
  const int p = pos[row];
  const float c = act ? rope_cos[static_cast<size_t>(p) * half + lane] : 0.f;
  const float s = act ? rope_sin[static_cast<size_t>(p) * half + lane] : 0.f;
  const int sl = is_q ? -1 : slot[row];
  float x0 = act ? sum(p0, col + lane) : 0.f;
  float x1 = act ? sum(p1, col + lane + half) : 0.f;
  if (gain) {
    const float ss = wave_sum(x0 * x0 + x1 * x1);
    const float inv = 1.0f / sqrtf(ss / static_cast<float>(d) + eps);
    if (act) {
      x0 = x0 * inv * g0;
      x1 = x1 * inv * g1;
    }
  }
  const float y0 = x0 * c - x1 * s;
  const float y1 = x1 * c + x0 * s;
  if (is_q) {
    if (act) {
      float* q = q_out + (static_cast<size_t>(row) * nq + h) * d;
      q[lane] = y0;
      q[lane + half] = y1;
    }
    return;
  }
  const int blk = sl >= 0 ? sl / kBlk : num_blocks - 1;
  const int off = sl >= 0 ? sl % kBlk : 0;
  if (act) {
    S* kp = static_cast<S*>(k_pool) + pool_k_at(blk, nkv, g, off, d);
    S* vp = static_cast<S*>(v_pool) + pool_v_at(blk, nkv, g, off, d);
    kp[lane] = T::from_f(y0);
    kp[lane + half] = T::from_f(y1);
    vp[lane * kBlk] = T::from_f(sum(pv0, vcol + lane));
    vp[(lane + half) * kBlk] = T::from_f(sum(pv1, vcol + lane + half));
  }
}

struct AttnRowsArgs {
  int nq, nkv;
  const float* q;            // [rows][nq][D] fp32 (prepared queries), or nullptr when fused below
  // fused decode prologue (q == nullptr): q, k from the QKV projection output (sum of n_parts
  // fp32 partials [rows][(nq + 2 nkv) D]), QK-RMSNorm + RoPE here; the split holding key L-1 of
  // a row writes the row's new K and V to its slot before any key of the split is read
  const float* qkv;
  int n_parts;
  size_t part_stride;
  const int* pos;
  const int* slot;
  const float* rope_cos;
  const float* rope_sin;
  const void* q_norm;
  const void* k_norm;
  float eps;
  void* k_pool;
  void* v_pool;
  const int* block_table;    // [reqs][bt_stride]
  int bt_stride;
  const int* row_ids;        // grid row -> row of q / out / seq_lens / row_req (nullptr: identity);
                             // a negative entry is an idle grid row. Partials are kept per grid row.
  const int* row_req;        // row -> block-table row (nullptr: identity)
  const int* seq_lens;       // [rows] keys visible to the row, its own token included
  int split_tokens;          // P: keys per split (multiple of 16)
  int max_splits;            // splits per row (gridDim.z, past which come prefetch blocks)
  int num_blocks;            // pool blocks; a negative table entry reads the scratch block
  void* out;                 // [rows][nq * D] in the model dtype
  float* partials;           // [rows][nq][max_splits][D + 2]: (max, sum, unnormalised output)
  unsigned* split_cnt;       // [grid rows][nkv] arrival counters, zero between launches: the last
                             // split of a (row, KV head) to finish merges the partials
  float scale;
  L2Prefetch pf;             // blocks with blockIdx.z >= max_splits only prefetch weights (pf.n > 0)
};

// Blocks past the split grid prefetch the weights of the GEMVs that follow (see l2_prefetch).
__device__ inline bool attn_prefetch_block(const AttnRowsArgs& a) {
  if (static_cast<int>(blockIdx.z) < a.max_splits) return false;
  const int plane = gridDim.x * gridDim.y;
  const int lin = blockIdx.x + gridDim.x * blockIdx.y + plane * blockIdx.z;
  l2_prefetch(a.pf, lin, plane * a.max_splits, plane * (gridDim.z - a.max_splits));
  return true;
}

constexpr int kMaxSplits = 128;   // splits per row one launch may use (the host sizes P for it)

// The split grid's live pieces, packed. The grid holds rows x nkv x max_splits blocks (fixed per
// bucket, so it replays as captured), but a row of L keys uses only ceil(L / P) splits (one, which
// writes zeros, when L <= 0; none for a padding row). The dispatcher hands consecutive blocks to
// the XCDs and CUs in turn, so in grid order the live blocks of a batch with a few long rows land
// on a few XCDs and pile up on shared CUs. With more than one split per row, block b instead takes
// the b-th live piece in (KV head, row, split) order, and blocks past the last one exit: every
// block counts the pieces of all rows (a block scan over the row table), then the thread whose
// rows hold piece b names it. Returns false for a block without a piece (block-uniform).
__device__ inline bool attn_piece(const AttnRowsArgs& a, int& prow, int& g, int& sp) {
  if (a.max_splits == 1) {   // one block per (row, KV head): the grid is already dense
    prow = blockIdx.x; g = blockIdx.y; sp = 0;
    return true;
  }
  __shared__ int s_w[4], s_piece[3];
  const int rows = gridDim.x, nkv = gridDim.y;
  const int b = blockIdx.x + rows * (blockIdx.y + nkv * blockIdx.z);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int per = (rows + 255) / 256;   // rows of this thread: [r0, r1)
  const int r0 = min(rows, threadIdx.x * per), r1 = min(rows, r0 + per);
  auto pieces = [&](int r) -> int {
    const int row = a.row_ids ? a.row_ids[r] : r;
    if (row < 0) return 0;
    const int L = a.seq_lens[row];
    return L <= 0 ? 1 : (L + a.split_tokens - 1) / a.split_tokens;
  };
  int mine = 0;
  for (int r = r0; r < r1; ++r) mine += pieces(r);
  int incl = mine;   // inclusive scan over the wave, then over the four waves
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) s_w[wid] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wid; ++w) before += s_w[w];
  const int total = s_w[0] + s_w[1] + s_w[2] + s_w[3];   // pieces of one KV head
  if (b >= nkv * total) return false;
  const int q = b % total;
  int at = incl - mine + before;   // first piece of this thread's rows
  if (q >= at && q < at + mine) {
    for (int r = r0; r < r1; ++r) {
      const int n = pieces(r);
      if (q < at + n) {
        s_piece[0] = r; s_piece[1] = b / total; s_piece[2] = q - at;
        break;
      }
      at += n;
    }
  }
  __syncthreads();
  prow = s_piece[0]; g = s_piece[1]; sp = s_piece[2];
  return true;
}

// RMSNorm over one head (optional gain) then rotate-half RoPE: lane holds the pair (lane, lane+D/2).
template <class T, int D>
__device__ inline void norm_rope_pair(float& x0, float& x1, const void* gain, float eps, float c, float s) {
  using S = typename T::S;
  constexpr int half = D / 2;
  const int lane = threadIdx.x & 63;
  const bool act = lane < half;
  if (gain) {
    const float ss = wave_sum(act ? x0 * x0 + x1 * x1 : 0.f);
    const float inv = 1.0f / sqrtf(ss / static_cast<float>(D) + eps);
    const S* gw = static_cast<const S*>(gain);
    if (act) {
      x0 = x0 * inv * T::to_f(gw[lane]);
      x1 = x1 * inv * T::to_f(gw[lane + half]);
    }
  }
  const float y0 = x0 * c - x1 * s;
  const float y1 = x1 * c + x0 * s;
  x0 = y0;
  x1 = y1;
}

// Queries of heads g*G .. g*G+G-1 of `row` into qs, scaled by 1/sqrt(D). With the fused decode
// prologue (a.q == nullptr) they are built from the QKV projection output here, and the split that
// holds key L-1 (holds_new) also writes the row's new K and V to its slot. Ends with a block barrier,
// so every key of the split is readable afterwards.
template <class T, int D, int G>
__device__ inline void attn_prologue(const AttnRowsArgs& a, int row, int g, bool holds_new, float (*qs)[D]) {
  using S = typename T::S;
  constexpr int half = D / 2;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (a.q) {
    for (int i = threadIdx.x; i < G * D; i += blockDim.x)
      qs[i / D][i % D] = a.q[(static_cast<size_t>(row) * a.nq + g * G) * D + i] * a.scale;
  } else {
    const int ld = (a.nq + 2 * a.nkv) * D;
    const int p = a.pos[row];
    const bool act = lane < half;
    const float c = act ? a.rope_cos[static_cast<size_t>(p) * half + lane] : 0.f;
    const float sn = act ? a.rope_sin[static_cast<size_t>(p) * half + lane] : 0.f;
    auto fetch = [&](int col) -> float {
      float v = 0.f;
      for (int k = 0; k < a.n_parts; ++k) v += a.qkv[k * a.part_stride + static_cast<size_t>(row) * ld + col];
      return v;
    };
    for (int j = wid; j < G; j += 4) {
      const int col = (g * G + j) * D;
      float x0 = act ? fetch(col + lane) : 0.f, x1 = act ? fetch(col + lane + half) : 0.f;
      norm_rope_pair<T, D>(x0, x1, a.q_norm, a.eps, c, sn);
      if (act) {
        qs[j][lane] = x0 * a.scale;
        qs[j][lane + half] = x1 * a.scale;
      }
    }
    if (holds_new && wid == 3) {
      // write the row's new K and V before any key of the split is read
      const int kcol = (a.nq + g) * D, vcol = (a.nq + a.nkv + g) * D;
      float k0 = act ? fetch(kcol + lane) : 0.f, k1 = act ? fetch(kcol + lane + half) : 0.f;
      norm_rope_pair<T, D>(k0, k1, a.k_norm, a.eps, c, sn);
      const int sl = a.slot[row];
      const int blk = sl >= 0 ? sl / kBlk : a.num_blocks - 1;
      const int off = sl >= 0 ? sl % kBlk : 0;
      if (act) {
        S* kp = static_cast<S*>(a.k_pool) + pool_k_at(blk, a.nkv, g, off, D);
        S* vp = static_cast<S*>(a.v_pool) + pool_v_at(blk, a.nkv, g, off, D);
        kp[lane] = T::from_f(k0);
        kp[lane + half] = T::from_f(k1);
        vp[lane * kBlk] = T::from_f(fetch(vcol + lane));
        vp[(lane + half) * kBlk] = T::from_f(fetch(vcol + lane + half));
      }
    }
  }
  __syncthreads();
}

// The fused decode prologue (a.q == nullptr) in two phases: attn_prologue_issue sends every load
// it needs (RoPE table entries, the first kPNP QKV partials of this wave's query heads and, in the
// wave that writes it, of the new key and value) before the split's key/value loads go out, and
// attn_prologue_finish does the sums (same order as attn_prologue, so the same bits), the norms,
// the rotation, the LDS and pool writes and the closing barrier while those loads are in flight.
constexpr int kPNP = 4;
template <int G>
struct PrologueRegs {
  static constexpr int HPW = (G + 3) / 4;   // query heads per wave
  float c = 0.f, sn = 0.f;
  float gq0 = 1.f, gq1 = 1.f, gk0 = 1.f, gk1 = 1.f;   // QK-norm gains of this lane's dims
  int slot = -1;
  float q[HPW][2][kPNP];
  float kv[4][kPNP];
};

// norm_rope_pair with the gain already in registers (the same arithmetic)
template <int D>
__device__ inline void norm_rope_pair_g(float& x0, float& x1, bool has_gain, float g0, float g1, float eps, float c,
                                        float s) {
  constexpr int half = D / 2;
  const bool act = static_cast<int>(threadIdx.x & 63) < half;
  if (has_gain) {
    const float ss = wave_sum(act ? x0 * x0 + x1 * x1 : 0.f);
    const float inv = 1.0f / sqrtf(ss / static_cast<float>(D) + eps);
    if (act) {
      x0 = x0 * inv * g0;
      x1 = x1 * inv * g1;
    }
  }
  const float y0 = x0 * c - x1 * s;
  const float y1 = x1 * c + x0 * s;
  x0 = y0;
  x1 = y1;
}

template <class T, int D, int G>
__device__ inline void attn_prologue_issue(const AttnRowsArgs& a, int row, int g, bool holds_new, PrologueRegs<G>& pr) {
  constexpr int half = D / 2;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const bool act = lane < half;
  const int p = a.pos[row];
  pr.c = act ? a.rope_cos[static_cast<size_t>(p) * half + lane] : 0.f;
  pr.sn = act ? a.rope_sin[static_cast<size_t>(p) * half + lane] : 0.f;
  using S = typename T::S;
  if (a.q_norm && act) {
    pr.gq0 = T::to_f(static_cast<const S*>(a.q_norm)[lane]);
    pr.gq1 = T::to_f(static_cast<const S*>(a.q_norm)[lane + half]);
  }
  const float* base = a.qkv + static_cast<size_t>(row) * (a.nq + 2 * a.nkv) * D;
  auto issue = [&](float(&dst)[kPNP], int col) {
#pragma unroll
    for (int k = 0; k < kPNP; ++k) dst[k] = (act && k < a.n_parts) ? base[k * a.part_stride + col] : 0.f;
  };
#pragma unroll
  for (int hh = 0; hh < PrologueRegs<G>::HPW; ++hh) {
    const int j = wid + 4 * hh;
    if (j < G) {
      issue(pr.q[hh][0], (g * G + j) * D + lane);
      issue(pr.q[hh][1], (g * G + j) * D + lane + half);
    }
  }
  if (holds_new && wid == 3) {
    const int kcol = (a.nq + g) * D, vcol = (a.nq + a.nkv + g) * D;
    pr.slot = a.slot[row];
    if (a.k_norm && act) {
      pr.gk0 = T::to_f(static_cast<const S*>(a.k_norm)[lane]);
      pr.gk1 = T::to_f(static_cast<const S*>(a.k_norm)[lane + half]);
    }
    issue(pr.kv[0], kcol + lane);
    issue(pr.kv[1], kcol + lane + half);
    issue(pr.kv[2], vcol + lane);
    issue(pr.kv[3], vcol + lane + half);
  }
}

template <class T, int D, int G>
__device__ inline void attn_prologue_finish(const AttnRowsArgs& a, int row, int g, bool holds_new,
                                            const PrologueRegs<G>& pr, float (*qs)[D]) {
  using S = typename T::S;
  constexpr int half = D / 2;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const bool act = lane < half;
  const float* base = a.qkv + static_cast<size_t>(row) * (a.nq + 2 * a.nkv) * D;
  // partials in order: the kPNP already loaded, then any further ones
  auto sum = [&](const float(&src)[kPNP], int col) -> float {
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < kPNP; ++k)
      if (k < a.n_parts) v += src[k];
    for (int k = kPNP; k < a.n_parts; ++k) v += base[k * a.part_stride + col];
    return v;
  };
#pragma unroll
  for (int hh = 0; hh < PrologueRegs<G>::HPW; ++hh) {
    const int j = wid + 4 * hh;
    if (j < G) {
      const int col = (g * G + j) * D;
      float x0 = act ? sum(pr.q[hh][0], col + lane) : 0.f, x1 = act ? sum(pr.q[hh][1], col + lane + half) : 0.f;
      norm_rope_pair_g<D>(x0, x1, a.q_norm != nullptr, pr.gq0, pr.gq1, a.eps, pr.c, pr.sn);
      if (act) {
        qs[j][lane] = x0 * a.scale;
        qs[j][lane + half] = x1 * a.scale;
      }
    }
  }
  if (holds_new && wid == 3) {
    // write the row's new K and V before any key of the split is read
    const int kcol = (a.nq + g) * D, vcol = (a.nq + a.nkv + g) * D;
    float k0 = act ? sum(pr.kv[0], kcol + lane) : 0.f, k1 = act ? sum(pr.kv[1], kcol + lane + half) : 0.f;
    norm_rope_pair_g<D>(k0, k1, a.k_norm != nullptr, pr.gk0, pr.gk1, a.eps, pr.c, pr.sn);
    const int sl = pr.slot;
    const int blk = sl >= 0 ? sl / kBlk : a.num_blocks - 1;
    const int off = sl >= 0 ? sl % kBlk : 0;
    if (act) {
      S* kp = static_cast<S*>(a.k_pool) + pool_k_at(blk, a.nkv, g, off, D);
      S* vp = static_cast<S*>(a.v_pool) + pool_v_at(blk, a.nkv, g, off, D);
      kp[lane] = T::from_f(k0);
      kp[lane + half] = T::from_f(k1);
      vp[lane * kBlk] = T::from_f(sum(pr.kv[2], vcol + lane));
      vp[(lane + half) * kBlk] = T::from_f(sum(pr.kv[3], vcol + lane + half));
    }
  }
  __syncthreads();
}

// Combine the four waves' (max, sum, unnormalised output) in wave order, then write the output
// (single split) or this split's partial. Call after a block barrier that follows the LDS writes.
template <class T, int D, int G>
__device__ inline void attn_finish(const AttnRowsArgs& a, int row, int prow, int g, int sp, int nsplit,
                                   const float (*wm)[G], const float (*wl)[G], const float (*wo)[G][D]) {
  using S = typename T::S;
  S* out = static_cast<S*>(a.out) + static_cast<size_t>(row) * a.nq * D;
  float* part = a.partials + (static_cast<size_t>(prow) * a.nq + g * G) * a.max_splits * (D + 2);
  for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
    const int j = i / D, dd = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, wm[w][j]);
    float Ls = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = (wm[w][j] == -INFINITY) ? 0.f : __expf(wm[w][j] - M);
      Ls += wl[w][j] * f;
      O += wo[w][j][dd] * f;
    }
    if (nsplit == 1) {
      out[(g * G + j) * D + dd] = T::from_f(O / Ls);
    } else {
      float* pp = part + (static_cast<size_t>(j) * a.max_splits + sp) * (D + 2);
      st_dev(pp + 2 + dd, O);
      if (dd == 0) { st_dev(pp, M); st_dev(pp + 1, Ls); }
    }
  }
  if (nsplit == 1) return;
  // The last split to arrive merges all splits in split order, so the result does not depend on
  // which split finished first. The partials go through device-scope stores and loads and one
  // device-scope counter per (row, KV head), reset by the merging block for the next launch.
  __shared__ int s_last;
  __shared__ float s_m[G][kMaxSplits], s_l[G][kMaxSplits];
  stores_done();
  __syncthreads();
  if (threadIdx.x == 0) s_last = arrive_last(a.split_cnt + static_cast<size_t>(prow) * a.nkv + g, nsplit);
  __syncthreads();
  if (!s_last) return;
  // One round of loads: the first kOB splits of each of the thread's NO output dims, and each
  // split's (max, sum) as one 8-byte load, all in flight together; then the sums in split order.
  // Block = 256 threads. (Fixed trip counts throughout: around a loop the compiler would drain the
  // outstanding loads first.)
  constexpr int NO = (G * D + 255) / 256;
  constexpr int kOB = NO == 1 ? 32 : (NO == 2 ? 16 : 8);
  constexpr int NML = (G * kMaxSplits + 255) / 256;
  const int nml = G * nsplit;
  const int tid = threadIdx.x;
  float ov[NO][kOB];
#pragma unroll
  for (int o = 0; o < NO; ++o) {
    const int i = tid + 256 * o;
    const bool act = i < G * D;
    const float* pj = part + static_cast<size_t>(act ? i / D : 0) * a.max_splits * (D + 2) + 2 + i % D;
#pragma unroll
    for (int k = 0; k < kOB; ++k) ov[o][k] = (act && k < nsplit) ? ld_dev(pj + static_cast<size_t>(k) * (D + 2)) : 0.f;
  }
  float2 mlv[NML];
#pragma unroll
  for (int r = 0; r < NML; ++r) {
    const int m = tid + 256 * r;
    if (m < nml) mlv[r] = ld_dev2(part + (static_cast<size_t>(m / nsplit) * a.max_splits + m % nsplit) * (D + 2));
  }
#pragma unroll
  for (int r = 0; r < NML; ++r) {
    const int m = tid + 256 * r;
    if (m < nml) { s_m[m / nsplit][m % nsplit] = mlv[r].x; s_l[m / nsplit][m % nsplit] = mlv[r].y; }
  }
  __syncthreads();
#pragma unroll
  for (int o = 0; o < NO; ++o) {
    const int i = tid + 256 * o;
    const bool act = i < G * D;
    const int j = act ? i / D : 0, dd = i % D;
    const float* pj = part + static_cast<size_t>(j) * a.max_splits * (D + 2) + 2 + dd;
    float M = -INFINITY;
    for (int s2 = 0; s2 < nsplit; ++s2) M = fmaxf(M, s_m[j][s2]);
    float Ls = 0.f, O = 0.f;
    for (int s0 = 0; s0 < nsplit; s0 += kOB) {
      if (s0) {
#pragma unroll
        for (int k = 0; k < kOB; ++k)
          ov[o][k] = (act && s0 + k < nsplit) ? ld_dev(pj + static_cast<size_t>(s0 + k) * (D + 2)) : 0.f;
      }
#pragma unroll
      for (int k = 0; k < kOB; ++k) {
        if (s0 + k < nsplit) {
          const float f = __expf(s_m[j][s0 + k] - M);
          Ls += s_l[j][s0 + k] * f;
          O += ov[o][k] * f;
        }
      }
    }
    if (act) out[(g * G + j) * D + dd] = T::from_f(O / Ls);
  }
}

// Attention with one query row per request ("One forward per step", section "What changed"),
// split over the key range so that short batches still fill the GPU (the same page, section
// "Bottleneck, and what follows"). Grid (rows, nkv, max_splits), whose blocks take the live (row,
// KV head, split) pieces in a packed order (attn_piece); split s of a row covers keys
// [s*P, min(seq_len, (s+1)*P)); blocks without a piece exit at once, so the grid depends on the
// bucket only and replays as captured. A row with one split writes its output; otherwise each
// split writes (max, sum, unnormalised output) and the last split to finish merges them in split
// order. Block = 4 waves; wave w takes the 16-key blocks w, w+4, ... of the split; the G = nq / nkv
// query heads sharing the KV head are processed together. Blocks past the split grid (z >=
// max_splits) only prefetch weights into L2. Two kernels share this contract: k_attn_rows_mfma
// (16-bit types, matrix cores) and k_attn_rows (any type, fp32 FMA; fp32 models).

// fp32 FMA version: 8 lanes per key in the score phase, a lane owns 8 dims in the value phase.
template <class T, int D, int G>
__global__ __launch_bounds__(256) void k_attn_rows(AttnRowsArgs a) {
  using S = typename T::S;
  constexpr int KL = D / 8;          // dims per lane in the score phase (8 lanes per key)
  constexpr int VG = 64 / (D / 8);   // key groups in the value phase (lane owns 8 dims)
  __shared__ float p_s[4][G][kBlk];
  __shared__ float wm[4][G], wl[4][G];
  __shared__ float wo[4][G][D];
  __shared__ float qs[G][D];
  if (attn_prefetch_block(a)) return;
  int prow, g, sp;
  if (!attn_piece(a, prow, g, sp)) return;
  const int row = a.row_ids ? a.row_ids[prow] : prow;
  if (row < 0) return;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int L = a.seq_lens[row];
  const int nsplit = (L + a.split_tokens - 1) / a.split_tokens;
  if (L <= 0) {
    if (sp == 0) {
      S* out = static_cast<S*>(a.out) + static_cast<size_t>(row) * a.nq * D;
      for (int i = threadIdx.x; i < G * D; i += blockDim.x) out[(g * G) * D + i] = T::from_f(0.f);
    }
    return;
  }
  if (sp >= nsplit) return;
  const int t0 = sp * a.split_tokens, t1 = min(L, t0 + a.split_tokens);
  const int req = a.row_req ? a.row_req[row] : row;
  const int* bt = a.block_table + static_cast<size_t>(req) * a.bt_stride;
  const int sub = lane & 7, kt = lane >> 3;
  const int vd = (lane % (D / 8)) * 8;  // value-phase dims of this lane
  const int vg = lane / (D / 8);        // value-phase key group
  const int nblk = (t1 - t0 + kBlk - 1) / kBlk;

  // K and V of one 16-key block, loaded straight into registers
  constexpr int KV16 = KL * sizeof(S) / 16;               // 16-byte vectors per lane per key pass
  uint4 kr[2][KV16 > 0 ? KV16 : 1];
  S vr[kBlk / VG][8];
  auto load_kv = [&](int bi) {
    const int tb = t0 + bi * kBlk;
    const int pb0 = (tb / kBlk < a.bt_stride) ? bt[tb / kBlk] : -1;
    const int pb = pb0 >= 0 ? pb0 : a.num_blocks - 1;
    const S* kp = static_cast<const S*>(a.k_pool) + pool_k_at(pb, a.nkv, g, 0, D);
    const S* vp = static_cast<const S*>(a.v_pool) + pool_v_at(pb, a.nkv, g, 0, D);
#pragma unroll
    for (int ps = 0; ps < 2; ++ps)
#pragma unroll
      for (int v = 0; v < KV16; ++v)
        kr[ps][v] = *reinterpret_cast<const uint4*>(kp + (ps * 8 + kt) * D + sub * KL + v * (16 / sizeof(S)));
#pragma unroll
    for (int i = 0; i < kBlk / VG; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) vr[i][e] = vp[(vd + e) * kBlk + vg + i * VG];
  };
  // The first block of this wave is loaded before the query prologue, unless it holds key L-1 of
  // a fused decode row (the prologue writes that key first).
  const bool holds_new = sp == nsplit - 1;
  const bool pre = (wid < nblk) && !(a.q == nullptr && holds_new && wid == nblk - 1);
  if (pre) load_kv(wid);
  attn_prologue<T, D, G>(a, row, g, holds_new, qs);

  // score-phase slice of this lane: dims (lane % 8) * KL .. + KL of each query head
  float q[G][KL];
#pragma unroll
  for (int j = 0; j < G; ++j)
#pragma unroll
    for (int e = 0; e < KL; ++e) q[j][e] = qs[j][sub * KL + e];

  float m[G], l[G], o[G][8];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[j][e] = 0.f;
  }
  for (int bi = wid; bi < nblk; bi += 4) {
    const int tb = t0 + bi * kBlk;                          // first key of the block
    if (bi != wid || !pre) load_kv(bi);

    // scores: 8 lanes per key, two passes of 8 keys
    float sc[2][G];
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
      float kf[KL];
#pragma unroll
      for (int v = 0; v < KV16; ++v) cvt_vec<T>(kr[ps][v], kf + v * T::kEPV);
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < KL; ++e) acc = fmaf(q[j][e], kf[e], acc);
        acc += __shfl_xor(acc, 1, 64);
        acc += __shfl_xor(acc, 2, 64);
        acc += __shfl_xor(acc, 4, 64);
        const int t = tb + ps * 8 + kt;
        sc[ps][j] = (t < t1) ? acc : -INFINITY;
      }
    }
    // block max per head over the 16 keys, new running max, probabilities
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float bm = fmaxf(sc[0][j], sc[1][j]);
      bm = fmaxf(bm, __shfl_xor(bm, 8, 64));
      bm = max_xor32(max_xor16(bm));
      const float mn = fmaxf(m[j], bm);
      const float corr = __expf(m[j] - mn);
      const float p0 = __expf(sc[0][j] - mn), p1 = __expf(sc[1][j] - mn);
      if (sub == 0) {
        p_s[wid][j][kt] = p0;
        p_s[wid][j][8 + kt] = p1;
      }
      float ps = p0 + p1;
      ps += __shfl_xor(ps, 8, 64);
      ps = add_xor32(add_xor16(ps));
      l[j] = l[j] * corr + ps;
      m[j] = mn;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[j][e] *= corr;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // values: lane owns dims vd .. vd+7 for keys vg, vg + VG, ...
#pragma unroll
    for (int i = 0; i < kBlk / VG; ++i) {
      // a masked key adds nothing, even if its slot holds NaN (0 * NaN would not be 0)
      const bool live = tb + vg + i * VG < t1;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float p = p_s[wid][j][vg + i * VG];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[j][e] = live ? fmaf(p, T::to_f(vr[i][e]), o[j][e]) : o[j][e];
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  // reduce the value accumulators over the key groups of the wave
#pragma unroll
  for (int j = 0; j < G; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      for (int off = D / 8; off < 64; off <<= 1) o[j][e] += __shfl_xor(o[j][e], off, 64);
  if (lane < D / 8) {
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) wo[wid][j][vd + e] = o[j][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < G; ++j) { wm[wid][j] = m[j]; wl[wid][j] = l[j]; }
  }
  __syncthreads();
  attn_finish<T, D, G>(a, row, prow, g, sp, nsplit, wm, wl, wo);
}

// Matrix-core version for 16-bit K/V (G <= 16 query heads per KV head). Per 16-key block a wave
// computes S^T[key][head] = K Q^T with v_mfma_f32_16x16x32 (K rows straight from the pool, Q^T
// rounded to the storage type and held in registers, columns past G zero), runs the online softmax
// on the accumulator (lane: keys 4*(l/16)+i of head l%16), and adds O^T[dim][head] += V^T P^T with
// v_mfma_f32_16x16x16, whose P^T operand is that accumulator rounded to the storage type and whose
// V^T operand is one 8-byte load of four consecutive keys from the dim-major V tile. A wave takes
// KB blocks per step (blocks b, b+4, ..., b+4(KB-1)) under one softmax update, so KB tiles are in
// flight at once; the next step's K is requested once the score products have issued and its V
// once the value products have. The block-table entries of the wave's blocks are fetched up front.
template <class T, int D, int G, int KB>
__global__ __launch_bounds__(256, KB == 1 ? 4 : 3) void k_attn_rows_mfma(AttnRowsArgs a) {
  using S = typename T::S;
  static_assert(sizeof(S) == 2 && G <= 16 && D % 32 == 0, "16-bit types, at most 16 heads per KV head");
  constexpr int KS = D / 32;   // k-steps of the score product
  constexpr int DT = D / 16;   // 16-dim tiles of the value product
  __shared__ __align__(16) float qs[G][D];
  __shared__ float wm[4][G], wl[4][G];
  __shared__ float wo[4][G][D];
  if (attn_prefetch_block(a)) return;
  int prow, g, sp;
  if (!attn_piece(a, prow, g, sp)) return;
  const int row = a.row_ids ? a.row_ids[prow] : prow;
  if (row < 0) return;
  const int lane = threadIdx.x & 63, wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int req = a.row_req ? a.row_req[row] : row;
  const int* bt = a.block_table + static_cast<size_t>(req) * a.bt_stride;
  const int t0 = sp * a.split_tokens;
  // table entries of this wave's blocks wid + 4k (lane k), fetched together with seq_len so that
  // no key load waits on a table load inside the loop
  const int bt_lane = t0 / kBlk + wid + 4 * lane;
  const int bt_pre = bt_lane < a.bt_stride ? bt[bt_lane] : -1;
  const int L = a.seq_lens[row];
  const int nsplit = (L + a.split_tokens - 1) / a.split_tokens;
  if (L <= 0) {
    if (sp == 0) {
      S* out = static_cast<S*>(a.out) + static_cast<size_t>(row) * a.nq * D;
      for (int i = threadIdx.x; i < G * D; i += blockDim.x) out[(g * G) * D + i] = T::from_f(0.f);
    }
    return;
  }
  if (sp >= nsplit) return;
  const int t1 = min(L, t0 + a.split_tokens);
  const int nblk = (t1 - t0 + kBlk - 1) / kBlk;

  uint4 kf[KB][KS];   // K fragment: key col, dims ks*32 + 8*grp .. + 8
  uint2 vf[KB][DT];   // V^T fragment: dim t*16 + col, keys 4*grp .. + 4
  // pool block of the split's block bi (scratch if unmapped or past the split)
  auto tile_of = [&](int bi) -> int {
    const int k = (bi - wid) / 4;       // wave-uniform
    int pb0 = -1;
    if (bi < nblk) {
      if (k < 64) {
        pb0 = __builtin_amdgcn_readlane(bt_pre, k);
      } else {
        const int tb = t0 + bi * kBlk;
        pb0 = (tb / kBlk < a.bt_stride) ? bt[tb / kBlk] : -1;
      }
    }
    return pb0 >= 0 ? pb0 : a.num_blocks - 1;
  };
  auto load_k = [&](int kb, int pb) {
    const S* kp = static_cast<const S*>(a.k_pool) + pool_k_at(pb, a.nkv, g, col, D) + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kf[kb][ks] = *reinterpret_cast<const uint4*>(kp + ks * 32);
  };
  auto load_v = [&](int kb, int pb) {
    const S* vp = static_cast<const S*>(a.v_pool) + pool_v_at(pb, a.nkv, g, 4 * grp, D) + col * kBlk;
#pragma unroll
    for (int t = 0; t < DT; ++t) vf[kb][t] = *reinterpret_cast<const uint2*>(vp + t * 16 * kBlk);
  };
  // The first step's blocks are loaded before the query prologue, except by the wave whose first
  // step holds the block of key L-1 of a fused decode row (the prologue writes that key first).
  const bool holds_new = sp == nsplit - 1;
  const int nb_new = nblk - 1 - wid;   // the new key's block, relative to this wave's first one
  const bool new_first = a.q == nullptr && holds_new && nb_new >= 0 && nb_new % 4 == 0 && nb_new / 4 < KB;
  const bool pre = (wid < nblk) && !new_first;
  // the fused prologue's own loads go out first, so its arithmetic overlaps the key/value loads
  PrologueRegs<G> pr;
  if (!a.q) attn_prologue_issue<T, D, G>(a, row, g, holds_new, pr);
  if (pre) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int pb = tile_of(wid + 4 * kb);
      load_k(kb, pb);
      load_v(kb, pb);
    }
  }
  if (a.q) attn_prologue<T, D, G>(a, row, g, holds_new, qs);
  else attn_prologue_finish<T, D, G>(a, row, g, holds_new, pr, qs);
  if (wid < nblk && !pre) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int pb = tile_of(wid + 4 * kb);
      load_k(kb, pb);
      load_v(kb, pb);
    }
  }
  // Q^T fragments: column = query head col (zero past G), k slots = dims ks*32 + 8*grp .. + 8
  uint4 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (col < G) {
      const float* src = &qs[col < G ? col : 0][ks * 32 + 8 * grp];
      qf[ks] = make_uint4(pack2<T>(src[0], src[1]), pack2<T>(src[2], src[3]), pack2<T>(src[4], src[5]),
                          pack2<T>(src[6], src[7]));
    } else {
      qf[ks] = make_uint4(0u, 0u, 0u, 0u);
    }
  }

  f32x4_t acc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;
  for (int b0 = wid; b0 < nblk; b0 += 4 * KB) {
    const bool more = b0 + 4 * KB < nblk;
    f32x4_t s[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      s[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s[kb] = mfma16x16x32<T>(kf[kb][ks], qf[ks], s[kb]);
    }
    if (more) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) load_k(kb, tile_of(b0 + 4 * KB + 4 * kb));
    }
    // this lane holds keys tb + 4*grp + i of head col (tb: first key of block b0 + 4kb); keys past
    // the split end, and blocks past the split, are masked
    float bm = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int tb = t0 + (b0 + 4 * kb) * kBlk;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[kb][i] = (tb + 4 * grp + i < t1) ? s[kb][i] : -INFINITY;
        bm = fmaxf(bm, s[kb][i]);
      }
    }
    bm = max_xor32(max_xor16(bm));
    const float mn = fmaxf(m, bm);                          // finite: block b0 has a live key
    const float corr = __expf(m - mn);
    float ps = 0.f;
    uint2 pt[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = __expf(s[kb][i] - mn);
        ps += p[i];
      }
      pt[kb] = make_uint2(pack2<T>(p[0], p[1]), pack2<T>(p[2], p[3]));
    }
    ps = add_xor32(add_xor16(ps));
    lsum = lsum * corr + ps;
    m = mn;
#pragma unroll
    for (int t = 0; t < DT; ++t) acc[t] *= corr;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int tb = t0 + (b0 + 4 * kb) * kBlk;
      if (tb + kBlk > t1) {
        // a masked key adds nothing, even if its slot holds NaN (0 * NaN would not be 0)
        const int k0 = tb + 4 * grp;
        const uint32_t m0 = (k0 < t1 ? 0xffffu : 0u) | (k0 + 1 < t1 ? 0xffff0000u : 0u);
        const uint32_t m1 = (k0 + 2 < t1 ? 0xffffu : 0u) | (k0 + 3 < t1 ? 0xffff0000u : 0u);
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          vf[kb][t].x &= m0;
          vf[kb][t].y &= m1;
        }
      }
#pragma unroll
      for (int t = 0; t < DT; ++t) acc[t] = mfma16x16x16<T>(vf[kb][t], pt[kb], acc[t]);
    }
    if (more) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) load_v(kb, tile_of(b0 + 4 * KB + 4 * kb));
    }
  }
  // per-wave state of head col: rows 4*grp + i of each 16-dim tile t
  if (col < G) {
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) wo[wid][col < G ? col : 0][t * 16 + 4 * grp + i] = acc[t][i];
    if (grp == 0) {
      wm[wid][col < G ? col : 0] = m;
      wl[wid][col < G ? col : 0] = lsum;
    }
  }
  __syncthreads();
  attn_finish<T, D, G>(a, row, prow, g, sp, nsplit, wm, wl, wo);
}


// ------------------------------------------------------------------------------------------------
// Balanced decode attention for many rows. The split grid above gives each (row, KV head, split) a
// block, so a launch lasts as long as its longest row: with rows of 16 to 4,352 keys most CUs sit
// idle for the last part of it, and many short rows leave many blocks with little to read. Here
// the launch's keys are cut into equal shares instead: the 16-key tiles of every (row, KV head)
// pair, taken in (row, KV head, tile) order, split into one contiguous share per wave, whatever
// the rows' lengths (the split-KV reading of "One forward per step", section "Bottleneck, and what
// follows": the split exists to fill the GPU, so it follows the keys, not the rows). A wave runs
// alone over its share: for each (row, KV head) piece it holds, the queries (and, in the piece
// holding key L-1 of a fused decode row, the new K and V), the tiles of the piece in order with
// KB tiles per online-softmax step, then the output (a whole pair) or the piece's (max, sum,
// unnormalised output) partial, of which the last-arriving wave merges the pair's pieces in piece
// order. Every block derives the same shares from the rows' lengths, so the grid is fixed and a
// captured launch replays at any lengths. It serves decode steps (one query row per request, the
// row's QK-norm + RoPE + KV write fused in as above). Split points follow the whole launch's
// lengths, so a row's output can change in its last bits with the other rows' lengths; rows
// without keys (the padding of a bucket) add no tiles and change nothing.
//
// Blocks per launch: two per CU of an MI355X (eight waves per CU; the kernel's registers allow two
// blocks per CU). Against one per CU, the second block's waves stream while the first's wait at a
// piece boundary: batch 256 (contexts 16-4,352) 328 -> 306 us per layer.
constexpr int kFlatBlocks = 512;
constexpr int kFlatWaves = 4 * kFlatBlocks;       // shares per launch at most
constexpr int kFlatMaxRows = 1024;                // grid rows the block-wide prefix sums hold
constexpr int kFlatMaxPieces = 64;                // waves one (row, KV head) pair may span (one lane each in the merge)
constexpr int kFlatMinTiles = 2;                  // smallest share, in 16-key tiles

// Partial slots of G query heads a flat launch over `rows` grid rows may use. Shares and pairs are
// both laid out in flat order, so the (wave, pair) intersections form a monotone path and wave +
// pair index names each one: at most kFlatWaves + rows * nkv slots.
__host__ __device__ inline long flat_slots(int rows, int nkv) {
  return static_cast<long>(kFlatWaves) + static_cast<long>(rows) * nkv;
}

template <class T, int D, int G, int KB>
__global__ __launch_bounds__(256, 2) void k_attn_flat(AttnRowsArgs a, int R) {
  using S = typename T::S;
  static_assert(sizeof(S) == 2 && G <= 8 && D % 32 == 0 && D <= 128, "16-bit types, at most 8 heads per KV head");
  constexpr int KS = D / 32;   // k-steps of the score product
  constexpr int DT = D / 16;   // 16-dim tiles of the value product
  constexpr int half = D / 2;
  constexpr int RPT = kFlatMaxRows / 256;
  __shared__ int pre[kFlatMaxRows + 1];   // first tile (per KV head) of each grid row
  __shared__ int red[2][4];
  __shared__ __align__(16) float qsw[4][G][D];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int nkv = a.nkv;

  // tiles of each row (0 for a row without keys), their prefix sums, the most
  int n[RPT], loc = 0, mx = 0;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int p = tid * RPT + i;
    const int L = p < R ? a.seq_lens[p] : 0;
    n[i] = L > 0 ? (L + kBlk - 1) / kBlk : 0;
    loc += n[i];
    mx = max(mx, n[i]);
  }
  int inc = loc;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(inc, o, 64);
    if (lane >= o) inc += v;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = max(mx, __shfl_xor(mx, o, 64));
  if (lane == 63) red[0][wid] = inc;
  if (lane == 0) red[1][wid] = mx;
  __syncthreads();
  int excl = inc - loc;
  for (int w = 0; w < wid; ++w) excl += red[0][w];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    pre[tid * RPT + i] = excl;
    excl += n[i];
  }
  if (tid == 255) pre[kFlatMaxRows] = excl;
  const int maxn = max(max(red[1][0], red[1][1]), max(red[1][2], red[1][3]));
  __syncthreads();
  // no block barrier from here on: the waves run independently
  const int gw = blockIdx.x * 4 + wid, NW = gridDim.x * 4;
  // rows without keys get a zero output
  for (int p = gw; p < R; p += NW) {
    if (pre[p + 1] != pre[p]) continue;
    S* out = static_cast<S*>(a.out) + static_cast<size_t>(p) * a.nq * D;
    for (int i = lane; i < a.nq * D; i += 64) out[i] = T::from_f(0.f);
  }
  const long total = static_cast<long>(nkv) * pre[kFlatMaxRows];
  if (total == 0) return;
  // Active waves: shares of at least kFlatMinTiles tiles, and no pair spread over more than
  // kFlatMaxPieces of them (a share of at least maxn / (kFlatMaxPieces - 2) tiles: a pair of n <=
  // maxn tiles then meets at most n / share + 2 shares).
  long nwa = NW;
  nwa = min(nwa, max(1L, total / kFlatMinTiles));
  nwa = min(nwa, max(1L, static_cast<long>(kFlatMaxPieces - 2) * total / (maxn + kFlatMaxPieces - 2)));
  if (gw >= nwa) return;
  auto wave_of = [&](long x) -> long { return ((x + 1) * nwa - 1) / total; };   // share holding flat tile x
  long f = static_cast<long>(gw) * total / nwa;
  const long f1 = static_cast<long>(gw + 1) * total / nwa;
  const int ld = (a.nq + 2 * nkv) * D;
  const bool act = lane < half;
  while (f < f1) {
    // the pair holding flat tile f: the last grid row whose first tile is at or before f (a row
    // with tiles, as f < total), then the KV head and the tile within the row's KV-head range
    int lo = 0, hi = R - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (static_cast<long>(nkv) * pre[mid] <= f) lo = mid;
      else hi = mid - 1;
    }
    const int row = __builtin_amdgcn_readfirstlane(lo);
    const int nr = __builtin_amdgcn_readfirstlane(pre[row + 1] - pre[row]);
    const long rbase = static_cast<long>(nkv) * pre[row];
    const int g = __builtin_amdgcn_readfirstlane(static_cast<int>((f - rbase) / nr));
    const int ta = __builtin_amdgcn_readfirstlane(static_cast<int>((f - rbase) % nr));
    const long seg0 = rbase + static_cast<long>(g) * nr;
    const int tb = static_cast<int>(min(static_cast<long>(nr), ta + (f1 - f)));
    f += tb - ta;
    const long fw = wave_of(seg0);
    const int np = static_cast<int>(wave_of(seg0 + nr - 1) - fw + 1);
    const int piece = static_cast<int>(gw - fw);
    const long slot0 = fw + static_cast<long>(row) * nkv + g;   // slot of piece 0 (see flat_slots)
    const int L = a.seq_lens[row];
    const int* bt = a.block_table + static_cast<size_t>(row) * a.bt_stride;
    const int nt = tb - ta;                       // tiles of the piece
    const int k1 = min(L, tb * kBlk);             // its keys: [ta * 16, k1)
    const bool writes_new = tb == nr;             // holds key L - 1: writes the row's new K and V
    // table entries of the piece's first 64 tiles, one per lane (later ones are read as needed)
    const int bt_pre = (lane < nt && ta + lane < a.bt_stride) ? bt[ta + lane] : -1;
    auto tile_of = [&](int i) -> int {            // i wave-uniform; past the piece: the scratch block
      int pb0 = -1;
      if (i < nt) {
        if (i < 64) pb0 = __builtin_amdgcn_readlane(bt_pre, i);
        else pb0 = (ta + i < a.bt_stride) ? bt[ta + i] : -1;
      }
      return pb0 >= 0 ? pb0 : a.num_blocks - 1;
    };
    uint4 kf[KB][KS];   // K fragment: key col, dims ks*32 + 8*grp .. + 8
    uint2 vf[KB][DT];   // V^T fragment: dim t*16 + col, keys 4*grp .. + 4
    auto load_k = [&](int kb, int pb) {
      const S* kp = static_cast<const S*>(a.k_pool) + pool_k_at(pb, nkv, g, col, D) + 8 * grp;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kf[kb][ks] = *reinterpret_cast<const uint4*>(kp + ks * 32);
    };
    auto load_v = [&](int kb, int pb) {
      const S* vp = static_cast<const S*>(a.v_pool) + pool_v_at(pb, nkv, g, 4 * grp, D) + col * kBlk;
#pragma unroll
      for (int t = 0; t < DT; ++t) vf[kb][t] = *reinterpret_cast<const uint2*>(vp + t * 16 * kBlk);
    };
    auto load_batch = [&](int i0) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int pb = tile_of(i0 + kb);
        load_k(kb, pb);
        load_v(kb, pb);
      }
    };
    // Queries: the prologue's loads go out first, then (unless the piece writes the new key,
    // which must reach the pool before its tile is read) the first tiles, so that the arithmetic
    // below overlaps those loads.
    float xq[G][2];
    float c = 0.f, sn = 0.f, gq0 = 1.f, gq1 = 1.f, gk0 = 1.f, gk1 = 1.f;
    float kv[4][kPNP];
    int slot = -1;
    const float* base = a.qkv + static_cast<size_t>(row) * ld;
    {
      float qp[G][2][kPNP];
#pragma unroll
      for (int j = 0; j < G; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int k = 0; k < kPNP; ++k)
            qp[j][h][k] = (act && k < a.n_parts) ? base[k * a.part_stride + (g * G + j) * D + lane + h * half] : 0.f;
      const int p = a.pos[row];
      c = act ? a.rope_cos[static_cast<size_t>(p) * half + lane] : 0.f;
      sn = act ? a.rope_sin[static_cast<size_t>(p) * half + lane] : 0.f;
      if (a.q_norm && act) {
        gq0 = T::to_f(static_cast<const S*>(a.q_norm)[lane]);
        gq1 = T::to_f(static_cast<const S*>(a.q_norm)[lane + half]);
      }
      if (writes_new) {
        const int kcol = (a.nq + g) * D, vcol = (a.nq + nkv + g) * D;
        slot = a.slot[row];
        if (a.k_norm && act) {
          gk0 = T::to_f(static_cast<const S*>(a.k_norm)[lane]);
          gk1 = T::to_f(static_cast<const S*>(a.k_norm)[lane + half]);
        }
#pragma unroll
        for (int k = 0; k < kPNP; ++k) {
          const bool on = act && k < a.n_parts;
          kv[0][k] = on ? base[k * a.part_stride + kcol + lane] : 0.f;
          kv[1][k] = on ? base[k * a.part_stride + kcol + lane + half] : 0.f;
          kv[2][k] = on ? base[k * a.part_stride + vcol + lane] : 0.f;
          kv[3][k] = on ? base[k * a.part_stride + vcol + lane + half] : 0.f;
        }
      } else {
        load_batch(0);
      }
      // partials summed in order: the kPNP loaded above, then any further ones
#pragma unroll
      for (int j = 0; j < G; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int cc = (g * G + j) * D + lane + h * half;
          float v = 0.f;
#pragma unroll
          for (int k = 0; k < kPNP; ++k)
            if (k < a.n_parts) v += qp[j][h][k];
          for (int k = kPNP; k < a.n_parts; ++k) v += act ? base[k * a.part_stride + cc] : 0.f;
          xq[j][h] = act ? v : 0.f;
        }
#pragma unroll
      for (int j = 0; j < G; ++j) norm_rope_pair_g<D>(xq[j][0], xq[j][1], a.q_norm != nullptr, gq0, gq1, a.eps, c, sn);
    }
    if (act) {
#pragma unroll
      for (int j = 0; j < G; ++j) {
        qsw[wid][j][lane] = xq[j][0] * a.scale;
        qsw[wid][j][lane + half] = xq[j][1] * a.scale;
      }
    }
    if (writes_new) {
      // the row's new K and V to its slot, complete before any tile of the piece is requested
      const int kcol = (a.nq + g) * D, vcol = (a.nq + nkv + g) * D;
      auto sum = [&](const float(&src)[kPNP], int cc) -> float {
        float v = 0.f;
#pragma unroll
        for (int k = 0; k < kPNP; ++k)
          if (k < a.n_parts) v += src[k];
        for (int k = kPNP; k < a.n_parts; ++k) v += base[k * a.part_stride + cc];
        return v;
      };
      float k0 = act ? sum(kv[0], kcol + lane) : 0.f, k1v = act ? sum(kv[1], kcol + lane + half) : 0.f;
      norm_rope_pair_g<D>(k0, k1v, a.k_norm != nullptr, gk0, gk1, a.eps, c, sn);
      const int blk = slot >= 0 ? slot / kBlk : a.num_blocks - 1;
      const int off = slot >= 0 ? slot % kBlk : 0;
      if (act) {
        S* kp = static_cast<S*>(a.k_pool) + pool_k_at(blk, nkv, g, off, D);
        S* vp = static_cast<S*>(a.v_pool) + pool_v_at(blk, nkv, g, off, D);
        kp[lane] = T::from_f(k0);
        kp[lane + half] = T::from_f(k1v);
        vp[lane * kBlk] = T::from_f(sum(kv[2], vcol + lane));
        vp[(lane + half) * kBlk] = T::from_f(sum(kv[3], vcol + lane + half));
      }
      stores_done();
      load_batch(0);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // Q^T fragments: column = query head col (zero past G), k slots = dims ks*32 + 8*grp .. + 8
    uint4 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (col < G) {
        const float* src = &qsw[wid][col < G ? col : 0][ks * 32 + 8 * grp];
        qf[ks] = make_uint4(pack2<T>(src[0], src[1]), pack2<T>(src[2], src[3]), pack2<T>(src[4], src[5]),
                            pack2<T>(src[6], src[7]));
      } else {
        qf[ks] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
    f32x4_t acc[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, lsum = 0.f;
    for (int i0 = 0; i0 < nt; i0 += KB) {
      const bool more = i0 + KB < nt;
      f32x4_t s[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        s[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) s[kb] = mfma16x16x32<T>(kf[kb][ks], qf[ks], s[kb]);
      }
      if (more) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) load_k(kb, tile_of(i0 + KB + kb));
      }
      // this lane holds keys t0 + 4*grp + i of head col (t0: first key of tile i0 + kb); keys past
      // the piece's end, and tiles past the piece, are masked
      float bm = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int t0 = (ta + i0 + kb) * kBlk;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s[kb][i] = (t0 + 4 * grp + i < k1) ? s[kb][i] : -INFINITY;
          bm = fmaxf(bm, s[kb][i]);
        }
      }
      bm = max_xor32(max_xor16(bm));
      const float mn = fmaxf(m, bm);                          // finite: tile i0 has a live key
      const float corr = __expf(m - mn);
      float ps = 0.f;
      uint2 pt[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        float pr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pr[i] = __expf(s[kb][i] - mn);
          ps += pr[i];
        }
        pt[kb] = make_uint2(pack2<T>(pr[0], pr[1]), pack2<T>(pr[2], pr[3]));
      }
      ps = add_xor32(add_xor16(ps));
      lsum = lsum * corr + ps;
      m = mn;
#pragma unroll
      for (int t = 0; t < DT; ++t) acc[t] *= corr;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int t0 = (ta + i0 + kb) * kBlk;
        if (t0 + kBlk > k1) {
          // a masked key adds nothing, even if its slot holds NaN (0 * NaN would not be 0)
          const int q0 = t0 + 4 * grp;
          const uint32_t m0 = (q0 < k1 ? 0xffffu : 0u) | (q0 + 1 < k1 ? 0xffff0000u : 0u);
          const uint32_t m1 = (q0 + 2 < k1 ? 0xffffu : 0u) | (q0 + 3 < k1 ? 0xffff0000u : 0u);
#pragma unroll
          for (int t = 0; t < DT; ++t) {
            vf[kb][t].x &= m0;
            vf[kb][t].y &= m1;
          }
        }
#pragma unroll
        for (int t = 0; t < DT; ++t) acc[t] = mfma16x16x16<T>(vf[kb][t], pt[kb], acc[t]);
      }
      if (more) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) load_v(kb, tile_of(i0 + KB + kb));
      }
    }
    S* out = static_cast<S*>(a.out) + (static_cast<size_t>(row) * a.nq + g * G) * D;
    if (np == 1) {   // the whole pair: its output (lane: dims t*16 + 4*grp + i of head col)
      if (col < G) {
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) out[col * D + t * 16 + 4 * grp + i] = T::from_f(acc[t][i] / lsum);
      }
      continue;
    }
    // this piece's partial, then the last of the pair's pieces to arrive merges them in piece order
    float* part = a.partials + static_cast<size_t>(slot0) * G * (D + 2);
    if (col < G) {
      float* pp = part + (static_cast<size_t>(piece) * G + col) * (D + 2);
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) st_dev(pp + 2 + t * 16 + 4 * grp + i, acc[t][i]);
      if (grp == 0) {
        st_dev(pp, m);
        st_dev(pp + 1, lsum);
      }
    }
    stores_done();
    int last = 0;
    if (lane == 0) last = arrive_last(a.split_cnt + static_cast<size_t>(row) * nkv + g, np) ? 1 : 0;
    if (!__builtin_amdgcn_readfirstlane(last)) continue;
    // lane p holds piece p's (max, sum) of each head: the pair's max, the pieces' factors, the total
    const bool live = lane < np;
    float fj[G], Lj[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float2 ml = live ? ld_dev2(part + (static_cast<size_t>(lane) * G + j) * (D + 2)) : make_float2(-INFINITY, 0.f);
      const float M = wave_max(ml.x);
      fj[j] = live ? __expf(ml.x - M) : 0.f;
      Lj[j] = wave_sum(fj[j] * ml.y);
    }
    constexpr int kMB = 8;   // pieces' loads in flight at once
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float* pj = part + static_cast<size_t>(j) * (D + 2) + 2;
      float o0 = 0.f, o1 = 0.f;
      for (int p0 = 0; p0 < np; p0 += kMB) {
        float v0[kMB], v1[kMB];
#pragma unroll
        for (int k = 0; k < kMB; ++k) {
          const size_t at = static_cast<size_t>(p0 + k) * G * (D + 2);
          v0[k] = (p0 + k < np && lane < D) ? ld_dev(pj + at + lane) : 0.f;
          v1[k] = (p0 + k < np && lane + 64 < D) ? ld_dev(pj + at + lane + 64) : 0.f;
        }
#pragma unroll
        for (int k = 0; k < kMB; ++k) {
          if (p0 + k < np) {
            const float fp = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fj[j]), p0 + k));
            o0 += fp * v0[k];
            o1 += fp * v1[k];
          }
        }
      }
      if (lane < D) out[j * D + lane] = T::from_f(o0 / Lj[j]);
      if (lane + 64 < D) out[j * D + lane + 64] = T::from_f(o1 / Lj[j]);
    }
  }
}

}  // namespace gr
