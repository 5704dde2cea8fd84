// One whole single-row decode step as ONE persistent kernel.
//
// "Removing overhead: fusion, graphs and async scheduling" (sections "Fewer, larger matmuls" and
// "CUDA graphs for a changing batch") and "Fast decode: syncs, CUDA graphs and compilation"
// (section "Where the time goes") trace batch-1 decode time to per-kernel overhead: a Qwen3-0.6B
// step is some 600 small launches, each too short to reach HBM bandwidth. A graph removes the host
// cost of those launches but not their device cost; on gfx950 every kernel boundary still costs its
// ramp-up, the HBM latency of its first weight loads, and a cache write-back. This kernel takes
// the pages' "fewer, larger kernels" to its end point for the batch-1 step: every layer runs inside
// one launch of one block per CU, and the kernel boundaries become device-side hand-offs.
//
// Hand-off. Values pass between phases as 8-byte words (fp32 value in the low half, a 32-bit tag
// in the high half) written and read with device-scope atomic stores and loads, so a word is
// either wholly old or wholly new. The consumer polls the data itself until every word it needs
// carries the tag of the (step, layer, phase) it waits for: one memory round trip per hand-off,
// with no separate flag or counter, and no cache-wide write-back or invalidate. The step's tags
// derive from an epoch word that the last block to finish advances, so words of earlier steps
// never match. A buffer is rewritten only after every reader of its previous contents has
// produced an output that the writer (transitively) waited for, so one buffer per phase suffices.
//
// Two roles per block. A wave's vector-memory counter completes in order, so a wave cannot use
// the result of a poll before every load it issued earlier has returned. The weight stream and
// the polls therefore live in different waves: waves 0-3 (compute) hold the weights of the next
// phases in registers, issued one phase ahead, and do the dot products and the attention
// products; waves 4-7 (exchange) only poll, keep the residual row, and do the norms. The two
// meet at block barriers that wait for LDS traffic only, never for the weight loads in flight.
//
// Phases of layer l (the rows of a projection are spread over all compute waves: wave w of W
// takes rows w, w + W, ...):
//   P1  QKV: r += down(l-1) (every block keeps the whole residual row r, updated in the same
//       order everywhere), x = RMSNorm(r) * g_in rounded to the dtype, qkv = W_qkv x (+ b).
//   P2  attention: item (kv head g, key split s of 64 TPW keys): QK-RMSNorm + RoPE of the G query heads and
//       the key, the new K and V written to the paged pool by the split that holds them, and
//       the split's (max, sum, unnormalised output) per query head, on the matrix cores.
//   P2b merge: item (query head h, 32-dim chunk c) combines the splits in split order ->
//       attention output (dtype).
//   P3  O projection.    P4  r += o; x = RMSNorm(r) * g_post; act = SiLU(gate) * up.
//   P5  down projection.
// After the last layer: r += down, final RMSNorm, the LM head over all waves -> fp32 logits.
//
// Every wait gives up after a bounded number of polls (or as soon as another wait has given up)
// and records where in *err, so the kernel always terminates; the host reads that word. All
// blocks must be resident at once: the host launches one block per CU (at most), and the kernel
// needs one block's resources per CU.
#pragma once
#include "attention.h"
#include "sample.h"

namespace gr {

// Keys per attention item: 64 * TPW, where TPW (the kernel's last template argument) is the number
// of 16-key tiles each of the four compute waves holds per item: 1 (64-key items) while a step's
// items fit one per block, 2 (128-key items) for rows twice as long.
constexpr int kPMaxSplits = 64;   // splits per KV head the merge stages in LDS
constexpr int kPSpin = 1 << 17;   // polls before a wait gives up (each poll is a memory round trip)
constexpr int kPPhases = 6;       // tagged phases per layer
constexpr int kPStamps = 512;     // timestamp slots (block 0, optional)
constexpr int kPThreads = 512;    // 4 compute waves + 4 exchange waves
constexpr int kPMaxLayers = 64;   // per-layer pointer table held in LDS
constexpr int kPMergeChunks = 4;  // merge items per query head (32 of the 128 dims each)
// Words that every block reads are written in kPReplicas copies, so that the 256 readers of a word
// spread over four lines instead of queueing on one. More copies cost the producers more stores
// than they save the readers: a 256-block all-to-all hand-off measured 1.35, 1.22, 1.19, 1.25 and
// 1.36 us with 1, 2, 4, 8 and 16 copies.
constexpr int kPReplicas = 4;
constexpr int kPRepStride = 4096 + 32;   // words between copies (>= the largest replicated buffer)
// Blocks per launch: one per CU of an MI355X. At this width every compute wave owns exactly one
// register tile of each projection at the widths the kernel is built for, and every attention item
// (at most kPBlocks of them) has a block of its own.
constexpr int kPBlocks = 256;

struct PLayer {
  const void *in_norm, *qkv_w, *qkv_b, *q_norm, *k_norm, *o_w, *post_norm, *gate_up_w, *down_w;
  void *k_pool, *v_pool;
};

struct PersistArgs {
  int layers, nq, nkv, vocab, max_position;
  float eps, scale;
  const PLayer* lw;                  // [layers], device memory
  const void *embed, *lm_head, *final_norm;
  int *ids, *pos, *slot, *len;       // row 0 of the decode metadata (advanced in place when sampling)
  const int* bt;
  int bt_stride, num_blocks, splits_alloc;
  const float *rope_cos, *rope_sin;
  uint64_t *x_qkv;                   // [(nq + 2 nkv) * 128]
  uint64_t *x_part;                  // [nq][splits_alloc][128 + 2]: max, sum, output
  // read by every block: kPReplicas copies kPRepStride words apart, block b reading copy b mod
  // kPReplicas
  uint64_t *x_attn;                  // [nq * 128 / 2] words of two values
  uint64_t *x_o, *x_down;            // [H]
  uint64_t *x_act;                   // [I / 3] words of three values
  unsigned* epoch;                   // advanced by the last block of each step
  unsigned* done;                    // arrival count, reset by the last block
  int* err;                          // 0, or the site where a wait gave up
  unsigned long long* stamps;        // optional [kPStamps] s_memrealtime stamps of block 0
  float* logits;                     // [vocab] row 0
  // Sampling fused into the LM head (sample != 0): the token the separate sampler would draw from
  // these logits (Gumbel-max with the same Philox uniforms; argmax at temperature 0), then the
  // same in-place advance of row 0 and of the step counter, by the last block.
  int sample;
  const float* temp;                 // [1] temperature
  uint64_t* rng;                     // {seed, step}
  uint64_t* cand;                    // [gridDim.x] each block's best (score key << 32 | ~index)
  int* tokens;                       // [1]
  int* history;                      // [max_position] or nullptr
};

__device__ inline void put_word(uint64_t* p, float v, uint32_t tag) {
  __hip_atomic_store(p, (static_cast<uint64_t>(tag) << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint64_t get_word(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Words of values already rounded to the 16-bit dtype carry more than one: two values and a 32-bit
// tag, or three values and the tag's low 16 bits. A 16-bit tag still tells the awaited write from
// the one before it (every word of such a buffer is rewritten at each of its phases, and
// consecutive tags differ by 6 or 7), which is the only other content a waiting reader can see.
__device__ inline void put_raw(uint64_t* p, uint64_t w) { __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ inline uint64_t word1(float v, uint32_t tag) { return (static_cast<uint64_t>(tag) << 32) | __float_as_uint(v); }
__device__ inline uint64_t word2(uint16_t v0, uint16_t v1, uint32_t tag) {
  return (static_cast<uint64_t>(tag) << 32) | static_cast<uint64_t>(v0) | (static_cast<uint64_t>(v1) << 16);
}
__device__ inline uint64_t word3(uint16_t v0, uint16_t v1, uint16_t v2, uint32_t tag) {
  return static_cast<uint64_t>(v0) | (static_cast<uint64_t>(v1) << 16) | (static_cast<uint64_t>(v2) << 32) |
         (static_cast<uint64_t>(tag & 0xffffu) << 48);
}
// a word of a replicated buffer, to every copy
__device__ inline void put_rep(uint64_t* base, int i, uint64_t w) {
#pragma unroll
  for (int r = 0; r < kPReplicas; ++r) put_raw(base + r * kPRepStride + i, w);
}
// this block's copy of a replicated buffer
__device__ inline const uint64_t* my_copy(const uint64_t* base) {
  return base + (blockIdx.x % kPReplicas) * kPRepStride;
}

// Block barrier that waits for this wave's LDS operations only; vector-memory loads in flight
// (the weights of later phases) stay in flight across it.
__device__ inline void bar() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Wait of the exchange waves for n tagged words: exchange thread t (0..255) takes the words
// i = t + 256 (B * round + b), b < B, whose address is addr(i), polls them until all carry `tag`
// (its low 16 bits in the top of the word with tag16), then passes each word to f(i, b, word).
// `sent` is the block's LDS word through which the watching wave releases the others.
template <int B, class Addr, class F>
__device__ inline void poll_words(int t, int n, uint32_t tag, int* err, int where, Addr&& addr, F&& f,
                                  volatile uint32_t* sent, bool tag16 = false) {
  const uint32_t tmask = tag16 ? 0xffffu : 0xffffffffu;
  const int tshift = tag16 ? 48 : 32;
  tag &= tmask;
  for (int i0 = t; i0 < n; i0 += 256 * B) {
    uint64_t v[B];
    // While the producers are still at work one lane of the block watches one word (the fewer
    // requests spin on the coherent lines, the sooner the others' stores show), and posts the tag
    // to LDS for the block's other exchange waves; then every lane reads all B until they carry
    // the tag. Blocks watch different words, so that no single line is polled by every CU.
    if (t < 64) {
      const int i = __builtin_amdgcn_readfirstlane((static_cast<int>(blockIdx.x) * 61) % n);
      for (int it = 0;; ++it) {
        uint32_t seen = 0;
        if (t == 0) seen = static_cast<uint32_t>(get_word(addr(i)) >> tshift) & tmask;
        if (__builtin_amdgcn_readfirstlane(seen) == tag) break;
        if ((it & 63) == 63) {
          if (it >= kPSpin) { atomicCAS(err, 0, where); break; }
          if (ld_dev(err) != 0) break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      if (t == 0) *sent = tag;
    } else {
      // a stale LDS value can only start the full read early; the full read checks every tag
      for (int it = 0;; ++it) {
        if (__builtin_amdgcn_readfirstlane(*sent) == tag) break;
        if ((it & 63) == 63) {
          if (it >= 64 * kPSpin) { atomicCAS(err, 0, where); break; }
          if (ld_dev(err) != 0) break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    for (int it = 0;; ++it) {
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const int i = i0 + 256 * b;
        v[b] = (i < n) ? get_word(addr(i)) : (static_cast<uint64_t>(tag) << tshift);
      }
      bool ok = true;
#pragma unroll
      for (int b = 0; b < B; ++b) ok &= (static_cast<uint32_t>(v[b] >> tshift) & tmask) == tag;
      if (ok) break;
      if ((it & 63) == 63) {
        if (it >= kPSpin) { atomicCAS(err, 0, where); break; }
        if (ld_dev(err) != 0) break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int i = i0 + 256 * b;
      if (i < n) f(i, b, v[b]);
    }
  }
}

template <class T>
__device__ inline float round_to(float x) { return T::to_f(T::from_f(x)); }
__device__ inline float word_f(uint64_t w) { return __uint_as_float(static_cast<uint32_t>(w)); }
__device__ inline uint16_t word_h(uint64_t w, int k) { return static_cast<uint16_t>(w >> (16 * k)); }

// Sum over the 64 lanes of a wave with data-parallel-primitive moves (a few cycles each, where a
// lane shuffle through LDS costs a round trip per step): quads, eights and rows of 16 in every
// lane, then the row broadcasts; lanes 48..63 end with the total, lane 63 is read.
template <int CTRL, int ROW_MASK>
__device__ inline float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}
__device__ inline float wave_sum63(float v) {
  v = dpp_add<0xb1, 0xf>(v);    // quad_perm [1, 0, 3, 2]
  v = dpp_add<0x4e, 0xf>(v);    // quad_perm [2, 3, 0, 1]
  v = dpp_add<0x141, 0xf>(v);   // row_half_mirror
  v = dpp_add<0x140, 0xf>(v);   // row_mirror
  v = dpp_add<0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
  v = dpp_add<0x143, 0xc>(v);   // row_bcast:31 into rows 2 and 3
  return v;
}

// the same moves for the maximum (lanes a move does not reach see -inf)
template <int CTRL, int ROW_MASK>
__device__ inline float dpp_max(float v) {
  return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(-INFINITY), __float_as_int(v), CTRL, ROW_MASK,
                                                             0xf, false)));
}
__device__ inline float wave_max63(float v) {
  v = dpp_max<0xb1, 0xf>(v);
  v = dpp_max<0x4e, 0xf>(v);
  v = dpp_max<0x141, 0xf>(v);
  v = dpp_max<0x140, 0xf>(v);
  v = dpp_max<0x142, 0xa>(v);
  v = dpp_max<0x143, 0xc>(v);
  return v;
}
// lane 63's value in every lane (a scalar read)
__device__ inline float lane63(float v) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63)); }

// Loads and stores through pointers the kernel reads from memory (the per-layer table) are
// generic; these make them global-memory accesses. A generic (flat) load also counts against
// the LDS counter, so every LDS access after it would wait for it.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
template <class V> struct NativeOf { using type = V; };
template <> struct NativeOf<uint4> { using type = u32x4_t; };
template <> struct NativeOf<uint2> { using type = u32x2_t; };
template <class V>
__device__ inline V ldg(const void* p, size_t i) {
  using N = typename NativeOf<V>::type;
  return __builtin_bit_cast(V, ((const __attribute__((address_space(1))) N*)(p))[i]);
}
template <class V>
__device__ inline void stg(void* p, size_t i, V v) {
  ((__attribute__((address_space(1))) V*)(p))[i] = v;
}

// acc + sum of the 8 products of two vectors of 8 packed 16-bit values
template <class T>
__device__ inline float dot8(const uint4& w, const uint4& x, float acc) {
  if constexpr (__is_same(T, BF16)) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.x), __builtin_bit_cast(bf16x2_t, x.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.y), __builtin_bit_cast(bf16x2_t, x.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.z), __builtin_bit_cast(bf16x2_t, x.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.w), __builtin_bit_cast(bf16x2_t, x.w), acc, false);
  } else {
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, w.x), __builtin_bit_cast(f16x2_t, x.x), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, w.y), __builtin_bit_cast(f16x2_t, x.y), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, w.z), __builtin_bit_cast(f16x2_t, x.z), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, w.w), __builtin_bit_cast(f16x2_t, x.w), acc, false);
  }
  return acc;
}

// The value, hidden from the optimiser: address arithmetic derived from it stays next to the loads
// that use it instead of being hoisted out of the layer loop, where the offsets of every load of
// every phase would stay live in registers for the whole step.
__device__ inline int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Weight rows of one GEMV phase held in registers: TR rows of this wave (row gw + NW * i for
// i = t * TR + r), NR = 2 pairs row j with row N + j (gate with up); VR 16-byte vectors per lane
// per row, lane l holding elements (v * 64 + l) * 8 .. + 8 of vector v (K = 512 * VR).
template <class T, int VR, int NR, int TR>
struct WTile {
  uint4 w[TR][NR][VR];
  float b[TR];
  // R >= 1 rows of this wave; past R the last row is loaded again (never used), so the number of
  // loads is fixed (the waits for them can then be counted exactly).
  __device__ inline void load(const void* W, const void* bias, int N, int gw, int NW, int R, int t) {
    using S = typename T::S;
    const int lane = opaque(static_cast<int>(threadIdx.x & 63));
    const int g0 = opaque(gw);
    constexpr int K = 512 * VR;
#pragma unroll
    for (int r = 0; r < TR; ++r) {
      const int i = min(t * TR + r, R - 1);
      const int row = g0 + NW * i;
#pragma unroll
      for (int h = 0; h < NR; ++h)
#pragma unroll
        for (int v = 0; v < VR; ++v)
          w[r][h][v] = ldg<uint4>(W, (static_cast<size_t>(row + h * N) * K + (v * 64 + lane) * 8) / 8);
      const float bv = T::to_f(ldg<S>(bias ? bias : W, bias ? row : 0));   // always a load: fixed count
      b[r] = bias ? bv : 0.f;
    }
  }
  // dot products of tile t with x (this lane's packed xv): epi(r, row, dot, paired dot) per
  // live row, valid in lane 63; two products per instruction (v_dot2c_f32_bf16 / _f16, fp32
  // accumulation)
  template <class Epi>
  __device__ inline void dot(const uint4 (&xv)[VR], int gw, int NW, int R, int t, Epi&& epi) const {
#pragma unroll
    for (int r = 0; r < TR; ++r) {
      const int i = t * TR + r;
      if (i >= R) break;
      float acc[NR];
#pragma unroll
      for (int h = 0; h < NR; ++h) {
        acc[h] = 0.f;
#pragma unroll
        for (int v = 0; v < VR; ++v) acc[h] = dot8<T>(w[r][h][v], xv[v], acc[h]);
      }
#pragma unroll
      for (int h = 0; h < NR; ++h) acc[h] = wave_sum63(acc[h]);
      epi(r, gw + NW * i, acc[0], acc[NR - 1]);   // the sums are in lane 63
    }
  }
};

// this lane's x values (8 packed 16-bit values per vector) for a VR-vector row layout, from the
// block's LDS copy
template <int VR>
__device__ inline void lane_x(const uint16_t* xs, uint4 (&xv)[VR]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int v = 0; v < VR; ++v) xv[v] = *reinterpret_cast<const uint4*>(xs + (v * 64 + lane) * 8);
}

// a value already rounded to the dtype, stored as its 16-bit pattern
template <class T>
__device__ inline uint16_t bits16(float x) { return __builtin_bit_cast(uint16_t, T::from_f(x)); }

// K and V tiles of one attention item: compute wave w takes the 16-key tiles w + 4 kb (kb < TPW)
// of the split (D = 128: K fragment 4 x 16 B, V^T fragment 8 x 8 B per tile, as in the decode
// attention kernel). Without an item (g < 0) the scratch block is loaded, so the load count is
// fixed.
template <int TPW>
struct AttnTiles {
  uint4 kf[TPW][4];
  uint2 vf[TPW][8];
};

// pool block of tile wid + 4 kb of split s (the scratch block where the split has no such tile);
// the same for every layer
template <int TPW>
__device__ inline int attn_tile_block(const PersistArgs& a, int g, int s, int L, int kb) {
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t0 = s * 64 * TPW;
  const int nblk = g < 0 ? 0 : (min(L, t0 + 64 * TPW) - t0 + kBlk - 1) / kBlk;
  const int bi = wid + 4 * kb;
  const int e = t0 / kBlk + bi;
  const int pb = (bi < nblk && e < a.bt_stride) ? a.bt[e] : -1;
  return __builtin_amdgcn_readfirstlane(pb >= 0 ? pb : a.num_blocks - 1);
}

template <int TPW>
__device__ inline void attn_tiles_load(AttnTiles<TPW>& at, const PersistArgs& a, const PLayer& lw, int g, const int (&pbs)[TPW]) {
  constexpr int D = 128;
  const int lane = opaque(static_cast<int>(threadIdx.x & 63));
  const int col = lane & 15, grp = lane >> 4;
  const int gg = g < 0 ? 0 : g;
#pragma unroll
  for (int kb = 0; kb < TPW; ++kb) {
    const int pb = pbs[kb];
    const size_t ko = pool_k_at(pb, a.nkv, gg, col, D) + 8 * grp;          // elements; multiple of 8
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) at.kf[kb][ks] = ldg<uint4>(lw.k_pool, (ko + ks * 32) / 8);
    const size_t vo = pool_v_at(pb, a.nkv, gg, 4 * grp, D) + col * kBlk;   // elements; multiple of 4
#pragma unroll
    for (int t = 0; t < 8; ++t) at.vf[kb][t] = ldg<uint2>(lw.v_pool, (vo + t * 16 * kBlk) / 4);
  }
}

// LDS of the attention phase
template <int G>
struct AttnLds {
  float stq[(G + 2) * 128];   // polled q heads, k, v of the item's KV head
  float qs[G][128];           // normed, rotated, scaled queries
  float kn[128];              // normed, rotated new key
  float wm[4][G], wl[4][G];
  float wo[4][G][128];
};

// Inputs of the attention items that do not depend on the step's data: RoPE at the row's
// position (the same for every layer) and a layer's QK-norm gains (exchange lane l: dims l and
// l + 64).
struct AttnConst {
  float c, sn, gq0, gq1, gk0, gk1;
};


// LDS of the step
template <int XS, int G>
struct PShared {
  uint16_t xs[2][XS];                  // normed / polled projection inputs (dtype bits), two in turn
  float red[4];                        // per-wave sums of squares of the exchange waves
  AttnLds<G> at;
  float mst[kPMaxSplits][130];         // merge: the splits of one query head
  // The per-layer pointers, copied from memory before any weight load is issued: a wave's loads
  // complete in order, so a table read from memory behind the weight loads in flight would wait
  // for all of them, where an LDS read does not.
  PLayer lw[kPMaxLayers];
  unsigned long long cand[8];          // per-wave sampling candidates
  uint32_t sent;                       // the tag the block's watching wave last saw
  int last;                            // this block is the last of the step to finish
};

// 1 / rms of the residual row from the exchange waves' partial sums of squares (after the barrier
// that follows norm_stage)
template <int XS, int G>
__device__ inline float norm_inv(const PShared<XS, G>& sh, int H, float eps) {
  return 1.0f / sqrtf((sh.red[0] + sh.red[1] + sh.red[2] + sh.red[3]) / static_cast<float>(H) + eps);
}

// Values every wave of a block derives the same way at the start of a step
struct PStep {
  int NB, tok, L, p, slot, nsplit, n_items;
  uint32_t tag0;
  float T;                 // sampling temperature, seed and Philox step counter
  uint64_t seed, stepc;
  __device__ uint32_t tag(int l, int ph) const { return tag0 + static_cast<uint32_t>(kPPhases * l + ph); }
};

__device__ inline void stamp(const PersistArgs& a, int k) {
  if (a.stamps && blockIdx.x == 0 && threadIdx.x == 256 && k < kPStamps) a.stamps[k] = __builtin_amdgcn_s_memrealtime();
}

// The barrier schedule of a step, shared by both roles: each role implements every stage (a
// stage a role has no part in is empty), so both roles pass the same barriers in the same order.
template <class Role>
__device__ inline void run_step(Role& ro, const PStep& st, int layers, int nq) {
  ro.start();
  for (int l = 0; l < layers; ++l) {
    ro.layer_start(l);
    ro.qkv_wait(l);              // P1
    ro.norm_stage(0);
    bar();
    stamp(ro.a, 1 + 8 * l);
    ro.qkv(l);
    if (static_cast<int>(blockIdx.x) < st.n_items) {   // P2: one item per block at most
      const int item = blockIdx.x;
      ro.attn_wait(l, item);
      bar();
      ro.attn_rope(l, item);
      bar();
      ro.attn_products(l, item);
      bar();
      ro.attn_partials(l, item);
      bar();
    }
    stamp(ro.a, 2 + 8 * l);
    for (int h = st.NB - 1 - static_cast<int>(blockIdx.x); h < nq * kPMergeChunks; h += st.NB) {   // P2b
      ro.merge_wait(l, h);
      bar();
      ro.merge(l, h);
      bar();
    }
    stamp(ro.a, 3 + 8 * l);
    ro.o_wait(l);                // P3
    bar();
    stamp(ro.a, 4 + 8 * l);
    ro.o_proj(l);
    ro.mlp_wait(l);              // P4
    ro.norm_stage(1);
    bar();
    stamp(ro.a, 5 + 8 * l);
    ro.gate_up(l);
    ro.down_wait(l);             // P5
    bar();
    stamp(ro.a, 6 + 8 * l);
    ro.down(l);
  }
  ro.final_wait();               // final norm + LM head
  ro.norm_stage(2);
  bar();
  stamp(ro.a, 1 + 8 * layers);
  ro.lm_head();
  stamp(ro.a, 2 + 8 * layers);
}

// Exchange role (waves 4-7): polls, the residual row, norms, QK-norm + RoPE, split merges.
template <class T, int VH, int VQ, int VI, int G>
struct ExchangeRole {
  using S = typename T::S;
  static constexpr int D = 128, H = 512 * VH, I = 512 * VI, RJ = H / 256, XS_ = 512 * (VI > VQ ? (VI > VH ? VI : VH) : (VQ > VH ? VQ : VH));
  const PersistArgs& a;
  const PStep& st;
  PShared<XS_, G>& sh;
  const int et, lane, wid;
  float r[RJ];                 // residual row, element et + 256 j
  float g[3][RJ];              // in_norm, post_norm, final_norm gains of the current layer
  AttnConst kc;
  bool qk = false;
  PLayer lw;

  __device__ ExchangeRole(const PersistArgs& a_, const PStep& s_, PShared<XS_, G>& sh_)
      : a(a_), st(s_), sh(sh_), et(static_cast<int>(threadIdx.x) - 256), lane(threadIdx.x & 63), wid(threadIdx.x >> 6) {}

  // the gains of layer l, requested right after a wait so that the next wait (which completes
  // only after every earlier load of the wave) finds them arrived
  __device__ void load_gains(int l) {
    constexpr int half = 64;
    const PLayer& nx = sh.lw[l];
#pragma unroll
    for (int j = 0; j < RJ; ++j) {
      g[0][j] = T::to_f(ldg<S>(nx.in_norm, et + 256 * j));
      g[1][j] = T::to_f(ldg<S>(nx.post_norm, et + 256 * j));
    }
    const bool q = nx.q_norm != nullptr;
    kc.gq0 = T::to_f(ldg<S>(q ? nx.q_norm : nx.in_norm, lane));
    kc.gq1 = T::to_f(ldg<S>(q ? nx.q_norm : nx.in_norm, lane + half));
    kc.gk0 = T::to_f(ldg<S>(q ? nx.k_norm : nx.in_norm, lane));
    kc.gk1 = T::to_f(ldg<S>(q ? nx.k_norm : nx.in_norm, lane + half));
  }
  __device__ void start() {
    constexpr int half = 64;
    const S* E = static_cast<const S*>(a.embed) + static_cast<size_t>(st.tok) * H;
#pragma unroll
    for (int j = 0; j < RJ; ++j) r[j] = T::to_f(E[et + 256 * j]);
    kc.c = a.rope_cos[static_cast<size_t>(st.p) * half + lane];
    kc.sn = a.rope_sin[static_cast<size_t>(st.p) * half + lane];
    load_gains(0);
  }
  __device__ void layer_start(int l) {
    lw = sh.lw[l];
    qk = lw.q_norm != nullptr;
  }
  __device__ void add_poll(const uint64_t* src, uint32_t tag, int where) {
    poll_words<RJ>(et, H, tag, a.err, where, [&](int i) { return src + i; }, [&](int, int b, uint64_t w) { r[b] += word_f(w); }, &sh.sent);
  }
  __device__ void qkv_wait(int l) {
    if (l > 0) add_poll(my_copy(a.x_down), st.tag(l - 1, 5), 6);
  }
  // RMSNorm in one barrier: the four waves' sums of squares of r go to red, and xs[0] gets
  // gain * r rounded to the dtype (gain 0: in_norm, 1: post_norm, 2: final_norm); the readers apply
  // RMSNorm's 1 / rms, a per-row scalar, to their dot products (W (g r / rms) = (W (g r)) / rms).
  __device__ void norm_stage(int which) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < RJ; ++j) ss += r[j] * r[j];
    ss = wave_sum63(ss);
    if (lane == 63) sh.red[wid - 4] = ss;
#pragma unroll
    for (int j = 0; j < RJ; ++j) {
      const float gn = which == 0 ? g[0][j] : which == 1 ? g[1][j] : g[2][j];
      sh.xs[0][et + 256 * j] = bits16<T>(r[j] * gn);
    }
  }
  __device__ void qkv(int) {}
  __device__ void attn_wait(int l, int item) {
    const int gq = item / st.nsplit;
    const int nq = a.nq, nkv = a.nkv;
    constexpr int BQ = ((G + 2) * 128 + 255) / 256;
    poll_words<BQ>(et, (G + 2) * D, st.tag(l, 0), a.err, 2, [&](int i) {
      const int h = i / D, d = i % D;
      const int c0 = (h < G) ? (gq * G + h) * D : (h == G ? (nq + gq) * D : (nq + nkv + gq) * D);
      return a.x_qkv + c0 + d;
    }, [&](int i, int, uint64_t w) { sh.at.stq[i] = word_f(w); }, &sh.sent);
  }
  __device__ void attn_rope(int, int) {
    constexpr int half = 64;
    for (int j = wid - 4; j <= G; j += 4) {
      float x0 = sh.at.stq[j * D + lane], x1 = sh.at.stq[j * D + lane + half];
      if (qk) {   // RMSNorm over the head with its gain, then rotate-half RoPE
        const float inv = 1.0f / sqrtf(lane63(wave_sum63(x0 * x0 + x1 * x1)) / static_cast<float>(D) + a.eps);
        x0 = x0 * inv * (j < G ? kc.gq0 : kc.gk0);
        x1 = x1 * inv * (j < G ? kc.gq1 : kc.gk1);
      }
      const float y0 = x0 * kc.c - x1 * kc.sn, y1 = x1 * kc.c + x0 * kc.sn;
      if (j < G) {
        sh.at.qs[j][lane] = y0 * a.scale;
        sh.at.qs[j][lane + half] = y1 * a.scale;
      } else {
        sh.at.kn[lane] = y0;
        sh.at.kn[lane + half] = y1;
      }
    }
  }
  __device__ void attn_products(int, int) {}
  __device__ void attn_partials(int, int) {}
  // merge item it = (query head it / 4, dims 32 (it % 4) .. + 32): each split's (max, sum) and
  // those 32 output dims, staged as mst[s][0, 1, 2 ..]
  __device__ void merge_wait(int l, int it) {
    constexpr int CW = D / kPMergeChunks, RW = CW + 2;   // dims per item, words per split
    const int h = it / kPMergeChunks, c = it % kPMergeChunks;
    const uint64_t* src = a.x_part + static_cast<size_t>(h) * a.splits_alloc * (D + 2);
    poll_words<3>(et, st.nsplit * RW, st.tag(l, 1), a.err, 3, [&](int i) {
      const int sp = i / RW, k = i % RW;
      return src + sp * (D + 2) + (k < 2 ? k : 2 + c * CW + (k - 2));
    }, [&](int i, int, uint64_t w) { sh.mst[i / RW][i % RW] = word_f(w); }, &sh.sent);
  }
  // the splits' partials -> attention output (dtype; zeros without keys), dims 2k and 2k + 1 of
  // head h in word h * 64 + k. Lane s holds split s's max and sum: the row's max, the splits'
  // rescale factors (back to LDS) and the total come from wave reductions; then the two half-waves
  // add the 32 dims over alternate splits, with the loads of several splits in flight at once.
  __device__ void merge(int l, int it) {
    constexpr int CW = D / kPMergeChunks;
    static_assert(kPMaxSplits <= 64 && CW == 32, "one split per lane; two half-waves of 32 dims");
    if (et >= 64) return;   // exchange wave 4
    const int h = it / kPMergeChunks, c = it % kPMergeChunks;
    const int ns = st.nsplit;
    float out = 0.f;
    if (ns > 0) {
      const bool live = lane < ns;
      const float ms = live ? sh.mst[lane][0] : -INFINITY;
      const float ls = live ? sh.mst[lane][1] : 0.f;
      const float M = lane63(wave_max63(ms));
      const float fs = live ? __expf(ms - M) : 0.f;
      const float Ls = lane63(wave_sum63(ls * fs));
      if (live) sh.mst[lane][1] = fs;   // a wave's LDS accesses complete in order
      const int d = lane & (CW - 1);
      float O = 0.f;
#pragma unroll 4
      for (int sp = lane >> 5; sp < ns; sp += 2) O += sh.mst[sp][2 + d] * sh.mst[sp][1];
      O = add_xor32(O);   // lanes l and l + 32: their two halves
      out = round_to<T>(O / Ls);
    }
    const float nb = __shfl_down(out, 1, 64);
    const int dim = c * CW + et;
    if (et < CW && (et & 1) == 0) put_rep(a.x_attn, h * (D / 2) + dim / 2, word2(bits16<T>(out), bits16<T>(nb), st.tag(l, 2)));
  }
  __device__ void o_wait(int l) {
    const uint64_t* src = my_copy(a.x_attn);
    poll_words<VQ>(et, a.nq * D / 2, st.tag(l, 2), a.err, 4, [&](int i) { return src + i; },
                   [&](int i, int, uint64_t w) {
                     sh.xs[1][2 * i] = word_h(w, 0);
                     sh.xs[1][2 * i + 1] = word_h(w, 1);
                   }, &sh.sent);
  }
  __device__ void o_proj(int) {}
  __device__ void mlp_wait(int l) { add_poll(my_copy(a.x_o), st.tag(l, 3), 5); }
  __device__ void gate_up(int) {}
  __device__ void down_wait(int l) {
    // word w holds act[w], act[w + I/3], act[w + 2 I/3] (the three gate|up rows of compute wave w)
    const uint64_t* src = my_copy(a.x_act);
    poll_words<(VI * 2 + 2) / 3>(et, I / 3, st.tag(l, 4), a.err, 7, [&](int i) { return src + i; },
                                 [&](int i, int, uint64_t w) {
                                   sh.xs[1][i] = word_h(w, 0);
                                   sh.xs[1][i + I / 3] = word_h(w, 1);
                                   sh.xs[1][i + 2 * (I / 3)] = word_h(w, 2);
                                 }, &sh.sent, true);
    if (l + 1 < a.layers) {
      load_gains(l + 1);
    } else {
#pragma unroll
      for (int j = 0; j < RJ; ++j) g[2][j] = T::to_f(static_cast<const S*>(a.final_norm)[et + 256 * j]);
    }
  }
  __device__ void down(int) {}
  __device__ void final_wait() { add_poll(my_copy(a.x_down), st.tag(a.layers - 1, 5), 8); }
  __device__ void lm_head();
};

// LM head rows of one wave: all eight waves of every block take rows gwl, gwl + NWL, ... in
// register tiles of TL rows, two tiles in turn (the next loading while one computes). The first
// tile is the caller's (the compute waves load it into their QKV tile during the last layer).
template <class T, int VH>
struct LmHead {
  static constexpr int TL = 4;
  using Tile = WTile<T, VH, 1, TL>;
  int gwl, NWL, R;
  __device__ void init(const PersistArgs& a) {
    gwl = blockIdx.x * 8 + (threadIdx.x >> 6);
    NWL = 8 * gridDim.x;
    R = (a.vocab - 1 - gwl) / NWL + 1;
  }
  __device__ void first(const PersistArgs& a, Tile& ta) const { ta.load(a.lm_head, nullptr, a.vocab, gwl, NWL, R, 0); }
  // the logits of this wave's rows; with sampling, the wave's best (score key, ~index) into *best
  __device__ void rest(const PersistArgs& a, const PStep& st, const uint16_t* xs, Tile& ta, float inv,
                       unsigned long long* best) const {
    Tile tb;
    const int lane = threadIdx.x & 63;
    uint4 xv[VH];
    lane_x<VH>(xs, xv);
    // lane j keeps the logits of the wave's rows j and j + 64 (the host keeps R <= 128)
    float z0 = 0.f, z1 = 0.f;
    int k = 0;
    auto epi = [&](int, int row, float y, float) {
      const float z = y * inv;
      if (lane == 63) a.logits[row] = z;
      const float zb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(z), 63));
      z0 = lane == k ? zb : z0;
      z1 = lane + 64 == k ? zb : z1;
      ++k;
    };
    const int nt = (R + TL - 1) / TL;
    for (int t = 0; t < nt; t += 2) {
      if (t + 1 < nt) tb.load(a.lm_head, nullptr, a.vocab, gwl, NWL, R, t + 1);
      ta.dot(xv, gwl, NWL, R, t, epi);
      if (t + 2 < nt) ta.load(a.lm_head, nullptr, a.vocab, gwl, NWL, R, t + 2);
      if (t + 1 < nt) tb.dot(xv, gwl, NWL, R, t + 1, epi);
    }
    if (!a.sample) return;
    // scores as the separate sampler forms them: z at temperature 0, else z / T plus Gumbel noise
    // of the (row 0, column) uniform; the largest key is the largest score, ties to the lowest index
    unsigned long long key = 0ull;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int i = lane + 64 * h;
      const int col = gwl + NWL * i;
      float sc = h ? z1 : z0;
      if (st.T > 0.f) sc = gumbel_score(sc / st.T, philox_uniform(st.seed, st.stepc, 0, col));
      const unsigned long long kk = (static_cast<unsigned long long>(fkey(sc)) << 32) | static_cast<uint32_t>(~col);
      key = (i < R && kk > key) ? kk : key;
    }
    key = wave_max_u64(key);
    if (lane == 0) *best = key;
  }
};

template <class T, int VH, int VQ, int VI, int G>
__device__ void ExchangeRole<T, VH, VQ, VI, G>::lm_head() {
  LmHead<T, VH> lm;
  lm.init(a);
  typename LmHead<T, VH>::Tile ta;
  lm.first(a, ta);
  lm.rest(a, st, sh.xs[0], ta, norm_inv(sh, H, a.eps), &sh.cand[threadIdx.x >> 6]);
}

// Compute role (waves 0-3): the projections' weights in registers, issued one phase ahead, their
// dot products, and the attention products on the matrix cores.
template <class T, int VH, int VQ, int VI, int G, int TPW>
struct ComputeRole {
  using S = typename T::S;
  static constexpr int D = 128, H = 512 * VH, I = 512 * VI, XS_ = 512 * (VI > VQ ? (VI > VH ? VI : VH) : (VQ > VH ? VQ : VH));
  static constexpr int TQ = 4, TO = 1, TG = 3, TD = 1;   // rows per register tile (one tile each at 256 blocks)
  static_assert(I == TG * 4 * kPBlocks, "the gate|up rows of a compute wave fill one packed word");
  static_assert(H <= kPRepStride && I / 3 <= kPRepStride && 512 * VQ / 2 <= kPRepStride, "replica stride");
  static_assert(TQ == LmHead<T, VH>::TL, "the QKV tile carries the first LM-head tile");
  const PersistArgs& a;
  const PStep& st;
  PShared<XS_, G>& sh;
  const int lane, wid, gw, NW, NQKV;
  int R_qkv, R_o, R_gu, R_dn;
  int g0, pbs[TPW];            // the block's attention item: KV head (-1: none), its tiles' pool blocks
  PLayer lw;
  WTile<T, VH, 1, TQ> wq;
  WTile<T, VQ, 1, TO> wo;
  WTile<T, VH, 2, TG> wg;
  WTile<T, VI, 1, TD> wd;
  AttnTiles<TPW> at;
  LmHead<T, VH> lm;

  __device__ ComputeRole(const PersistArgs& a_, const PStep& s_, PShared<XS_, G>& sh_)
      : a(a_), st(s_), sh(sh_), lane(threadIdx.x & 63), wid(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)),
        gw(blockIdx.x * 4 + wid),
        NW(4 * gridDim.x), NQKV((a_.nq + 2 * a_.nkv) * D) {
    auto rows_of = [&](int N) { return (N - 1 - gw) / NW + 1; };
    R_qkv = rows_of(NQKV); R_o = rows_of(H); R_gu = rows_of(I); R_dn = rows_of(H);
    lm.init(a);
  }
  // The block table is read before any weight load is in flight (a wave's loads complete in
  // order, so a table read behind them would wait for all of them).
  __device__ void start() {
    const int it = blockIdx.x;
    const bool has = it < st.n_items;
    g0 = has ? it / st.nsplit : -1;
    const int s0 = has ? it % st.nsplit : 0;
#pragma unroll
    for (int kb = 0; kb < TPW; ++kb) pbs[kb] = attn_tile_block<TPW>(a, g0, s0, st.L, kb);
    wq.load(sh.lw[0].qkv_w, sh.lw[0].qkv_b, NQKV, gw, NW, R_qkv, 0);
    attn_tiles_load(at, a, sh.lw[0], g0, pbs);
    wo.load(sh.lw[0].o_w, nullptr, H, gw, NW, R_o, 0);
  }
  // Weights (and attention tiles) go out two phases or more before their use, each batch after the
  // issuing phase's own outputs are stored (with the whole chip loading weights at once, issuing
  // loads can stall the wave until queue slots free up): gate|up after QKV, down after O, the next
  // layer's QKV after gate|up, its attention tiles and O after down. A block with an attention
  // item issues gate|up and down after its attention partials instead: its exchange waves are not
  // polling then, while a poll issued behind a weight burst on the CU waits for the burst. The
  // order keeps every wait exact or early: each use waits for its own batch and the older ones.
  __device__ void layer_start(int l) { lw = sh.lw[l]; }
  __device__ void qkv_wait(int) {}
  __device__ void norm_stage(int) {}
  __device__ void qkv(int l) {
    uint4 xv[VH];
    lane_x<VH>(sh.xs[0], xv);
    const uint32_t tg = st.tag(l, 0);
    const float inv = norm_inv(sh, H, a.eps);
    wq.dot(xv, gw, NW, R_qkv, 0, [&](int r, int row, float y, float) {
      if (lane == 63) put_word(a.x_qkv + row, y * inv + wq.b[r], tg);
    });
    // an attention block issues them after its attention products instead (its exchange waves are
    // about to wait for this step's q, k and v, and loads in flight on the CU would delay that wait)
    if (g0 < 0) wg.load(lw.gate_up_w, nullptr, I, gw, NW, R_gu, 0);
  }
  __device__ void attn_wait(int, int) {}   // the tiles of the block's (only) item went out at layer start
  __device__ void attn_rope(int, int) {}
  // the new K and V to the pool, key L - 1 patched into its tile, the products, per-wave state
  __device__ void attn_products(int, int item) {
    constexpr int half = 64;
    const int g = item / st.nsplit, s = item % st.nsplit;
    const int col = lane & 15, grp = lane >> 4;
    const int L = st.L;
    const int t0 = s * 64 * TPW, t1 = min(L, t0 + 64 * TPW);
    const int nblk = (t1 - t0 + kBlk - 1) / kBlk;
    const float* vnew = sh.at.stq + (G + 1) * D;
    if (s == st.nsplit - 1) {
      if (wid == 3) {
        const int sl = st.slot;
        const int blk = sl >= 0 ? sl / kBlk : a.num_blocks - 1;
        const int off = sl >= 0 ? sl % kBlk : 0;
        const size_t ko = pool_k_at(blk, a.nkv, g, off, D), vo = pool_v_at(blk, a.nkv, g, off, D);
        stg<S>(lw.k_pool, ko + lane, T::from_f(sh.at.kn[lane]));
        stg<S>(lw.k_pool, ko + lane + half, T::from_f(sh.at.kn[lane + half]));
        stg<S>(lw.v_pool, vo + lane * kBlk, T::from_f(vnew[lane]));
        stg<S>(lw.v_pool, vo + (lane + half) * kBlk, T::from_f(vnew[lane + half]));
      }
      const int bn = (L - 1 - t0) / kBlk, on = (L - 1) % kBlk;
      if ((bn & 3) == wid) {
        const int kb = bn >> 2;
#pragma unroll
        for (int q = 0; q < TPW; ++q) {
          if (q != kb) continue;
          if (col == on) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
              const float* src = sh.at.kn + ks * 32 + 8 * grp;
              at.kf[q][ks] = make_uint4(pack2<T>(src[0], src[1]), pack2<T>(src[2], src[3]), pack2<T>(src[4], src[5]),
                                        pack2<T>(src[6], src[7]));
            }
          }
          if (grp == (on >> 2)) {
            const int e = on & 3;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
              const uint32_t nv = pack2<T>(vnew[t * 16 + col], 0.f) & 0xffffu;
              uint32_t x = at.vf[q][t].x, y = at.vf[q][t].y;
              if (e == 0) x = (x & 0xffff0000u) | nv;
              else if (e == 1) x = (x & 0xffffu) | (nv << 16);
              else if (e == 2) y = (y & 0xffff0000u) | nv;
              else y = (y & 0xffffu) | (nv << 16);
              at.vf[q][t] = make_uint2(x, y);
            }
          }
        }
      }
    }
    // Q^T fragments: column = query head col (zero past G), k slots = dims ks*32 + 8*grp .. + 8
    uint4 qf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (col < G) {
        const float* src = &sh.at.qs[col < G ? col : 0][ks * 32 + 8 * grp];
        qf[ks] = make_uint4(pack2<T>(src[0], src[1]), pack2<T>(src[2], src[3]), pack2<T>(src[4], src[5]),
                            pack2<T>(src[6], src[7]));
      } else {
        qf[ks] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
    f32x4_t acc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, lsum = 0.f;
    if (wid < nblk) {
      f32x4_t sc[TPW];
#pragma unroll
      for (int kb = 0; kb < TPW; ++kb) {
        sc[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) sc[kb] = mfma16x16x32<T>(at.kf[kb][ks], qf[ks], sc[kb]);
      }
      float bm = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < TPW; ++kb) {
        const int tb = t0 + (wid + 4 * kb) * kBlk;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sc[kb][i] = (tb + 4 * grp + i < t1) ? sc[kb][i] : -INFINITY;
          bm = fmaxf(bm, sc[kb][i]);
        }
      }
      bm = max_xor32(max_xor16(bm));
      m = bm;                                                   // finite: tile wid has a live key
      float ps = 0.f;
      uint2 pt[TPW];
#pragma unroll
      for (int kb = 0; kb < TPW; ++kb) {
        float pr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pr[i] = __expf(sc[kb][i] - m);
          ps += pr[i];
        }
        pt[kb] = make_uint2(pack2<T>(pr[0], pr[1]), pack2<T>(pr[2], pr[3]));
      }
      ps = add_xor32(add_xor16(ps));
      lsum = ps;
#pragma unroll
      for (int kb = 0; kb < TPW; ++kb) {
        const int tb = t0 + (wid + 4 * kb) * kBlk;
        if (tb + kBlk > t1) {
          // a masked key adds nothing, even if its slot holds NaN (0 * NaN would not be 0)
          const int k0 = tb + 4 * grp;
          const uint32_t m0 = (k0 < t1 ? 0xffffu : 0u) | (k0 + 1 < t1 ? 0xffff0000u : 0u);
          const uint32_t m1 = (k0 + 2 < t1 ? 0xffffu : 0u) | (k0 + 3 < t1 ? 0xffff0000u : 0u);
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            at.vf[kb][t].x &= m0;
            at.vf[kb][t].y &= m1;
          }
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[t] = mfma16x16x16<T>(at.vf[kb][t], pt[kb], acc[t]);
      }
    }
    if (col < G) {
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) sh.at.wo[wid][col < G ? col : 0][t * 16 + 4 * grp + i] = acc[t][i];
      if (grp == 0) {
        sh.at.wm[wid][col < G ? col : 0] = m;
        sh.at.wl[wid][col < G ? col : 0] = lsum;
      }
    }
  }
  // the four compute waves' states in wave order -> this split's partial of each query head
  __device__ void attn_partials(int l, int item) {
    const int g = item / st.nsplit, s = item % st.nsplit;
    const uint32_t tg = st.tag(l, 1);
    for (int i = threadIdx.x; i < G * D; i += 256) {
      const int j = i / D, dd = i % D;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) M = fmaxf(M, sh.at.wm[w][j]);
      float Ls = 0.f, O = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = (sh.at.wm[w][j] == -INFINITY) ? 0.f : __expf(sh.at.wm[w][j] - M);
        Ls += sh.at.wl[w][j] * f;
        O += sh.at.wo[w][j][dd] * f;
      }
      uint64_t* pp = a.x_part + (static_cast<size_t>(g * G + j) * a.splits_alloc + s) * (D + 2);
      put_word(pp + 2 + dd, O, tg);
      if (dd == 0) {
        put_word(pp, M, tg);
        put_word(pp + 1, Ls, tg);
      }
    }
    wg.load(lw.gate_up_w, nullptr, I, gw, NW, R_gu, 0);
    wd.load(lw.down_w, nullptr, H, gw, NW, R_dn, 0);
  }
  __device__ void merge_wait(int, int) {}
  __device__ void merge(int, int) {}
  __device__ void o_wait(int) {}
  __device__ void o_proj(int l) {
    uint4 xv[VQ];
    lane_x<VQ>(sh.xs[1], xv);
    const uint32_t tg = st.tag(l, 3);
    wo.dot(xv, gw, NW, R_o, 0, [&](int, int row, float y, float) {
      if (lane == 63) put_rep(a.x_o, row, word1(y, tg));
    });
    if (g0 < 0) wd.load(lw.down_w, nullptr, H, gw, NW, R_dn, 0);   // attention blocks: after partials
  }
  __device__ void mlp_wait(int) {}
  __device__ void gate_up(int l) {
    uint4 xv[VH];
    lane_x<VH>(sh.xs[0], xv);
    const uint32_t tg = st.tag(l, 4);
    uint16_t act[TG];
    const float inv = norm_inv(sh, H, a.eps);
    wg.dot(xv, gw, NW, R_gu, 0, [&](int r, int, float gt, float up) { act[r] = bits16<T>(silu(gt * inv) * (up * inv)); });
    if (lane == 63) put_rep(a.x_act, gw, word3(act[0], act[1], act[2], tg));   // rows gw, gw + NW, gw + 2 NW
    // the next layer's QKV weights (or the first LM-head tile: same tile shape), through one load
    // sequence either way (the waits stay exact)
    const bool last = l + 1 == a.layers;
    const PLayer& nx = sh.lw[last ? l : l + 1];
    wq.load(last ? a.lm_head : nx.qkv_w, last ? nullptr : nx.qkv_b, last ? a.vocab : NQKV, last ? lm.gwl : gw,
            last ? lm.NWL : NW, last ? lm.R : R_qkv, 0);
  }
  __device__ void down_wait(int) {}
  // the next layer's attention tiles and O weights go out after the down products (after the last
  // layer: the same loads again, never used, so that the load sequence is the same every layer)
  __device__ void down(int l) {
    uint4 xv[VI];
    lane_x<VI>(sh.xs[1], xv);
    const uint32_t tg = st.tag(l, 5);
    wd.dot(xv, gw, NW, R_dn, 0, [&](int, int row, float y, float) {
      if (lane == 63) put_rep(a.x_down, row, word1(y, tg));
    });
    const PLayer& nx = sh.lw[l + 1 < a.layers ? l + 1 : l];
    attn_tiles_load(at, a, nx, g0, pbs);
    wo.load(nx.o_w, nullptr, H, gw, NW, R_o, 0);
  }
  __device__ void final_wait() {}
  __device__ void lm_head() { lm.rest(a, st, sh.xs[0], wq, norm_inv(sh, H, a.eps), &sh.cand[threadIdx.x >> 6]); }
};

// The step. VH, VQ, VI: 16-byte vectors per lane of a row of length H, nq * 128 and I (each a
// multiple of 512); G: query heads per KV head. Every compute wave must own at least one row of
// the QKV, O, gate|up and down phases and every wave one LM-head row (the host keeps 4 * gridDim.x
// <= the narrowest projection and 8 * gridDim.x <= the vocabulary).
template <class T, int VH, int VQ, int VI, int G, int TPW>
__global__ __launch_bounds__(kPThreads, 1) void k_persist_decode(PersistArgs a) {
  constexpr int XS = 512 * (VI > VQ ? (VI > VH ? VI : VH) : (VQ > VH ? VQ : VH));
  __shared__ __align__(16) PShared<XS, G> sh;
  const unsigned ep = __builtin_amdgcn_readfirstlane(__hip_atomic_load(a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  PStep st;
  st.NB = gridDim.x;
  st.tok = a.ids[0];
  st.L = a.len[0];
  st.p = min(max(a.pos[0], 0), a.max_position - 1);
  st.slot = a.slot[0];
  if (threadIdx.x == 0) sh.sent = 0u;
  st.T = a.sample ? a.temp[0] : 0.f;
  st.seed = a.sample ? a.rng[0] : 0ull;
  st.stepc = a.sample ? a.rng[1] : 0ull;
  {
    constexpr int kw = sizeof(PLayer) / sizeof(uint64_t);
    static_assert(sizeof(PLayer) % sizeof(uint64_t) == 0, "PLayer is a whole number of words");
    const uint64_t* src = reinterpret_cast<const uint64_t*>(a.lw);
    uint64_t* dst = reinterpret_cast<uint64_t*>(sh.lw);
    for (int i = threadIdx.x; i < a.layers * kw; i += kPThreads) dst[i] = src[i];
  }
  __syncthreads();
  st.nsplit = (st.L + 64 * TPW - 1) / (64 * TPW);
  st.n_items = a.nkv * st.nsplit;
  st.tag0 = (ep + 1u) * static_cast<uint32_t>(kPPhases * a.layers + 1);
  stamp(a, 0);
  if (threadIdx.x >= 256) {
    ExchangeRole<T, VH, VQ, VI, G> ro(a, st, sh);
    run_step(ro, st, a.layers, a.nq);
  } else {
    ComputeRole<T, VH, VQ, VI, G, TPW> ro(a, st, sh);
    run_step(ro, st, a.layers, a.nq);
  }
  // the last block to finish takes the token (when sampling) and advances the epoch for the next
  // step; every block read the step's inputs before it counted itself in
  stores_done();
  __syncthreads();
  if (threadIdx.x == 0) {
    if (a.sample) {
      unsigned long long b = sh.cand[0];
      for (int w = 1; w < 8; ++w) b = sh.cand[w] > b ? sh.cand[w] : b;
      put_raw(reinterpret_cast<uint64_t*>(a.cand) + blockIdx.x, b);
      stores_done();
    }
    sh.last = arrive_last(a.done, gridDim.x);
  }
  __syncthreads();
  if (!sh.last) return;
  // A wait that gave up (now or in an earlier step whose failure the host has not yet collected
  // with step_device_status) leaves this step's values undefined: the logits become NaN, the token
  // -1, and the row does not advance, so a replay loop cannot feed them forward. Every block's
  // stores completed before it counted itself in, so these stores come last.
  if (ld_dev(a.err) != 0) {
    for (int i = threadIdx.x; i < a.vocab; i += kPThreads) a.logits[i] = __builtin_nanf("");
    if (threadIdx.x == 0) {
      if (a.sample) a.tokens[0] = -1;
      __hip_atomic_store(a.epoch, ep + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }
  if (a.sample) {
    unsigned long long b = 0ull;
    for (int i = threadIdx.x; i < static_cast<int>(gridDim.x); i += kPThreads) {
      const unsigned long long w = get_word(a.cand + i);
      b = w > b ? w : b;
    }
    b = wave_max_u64(b);
    if ((threadIdx.x & 63) == 0) sh.cand[threadIdx.x >> 6] = b;
    __syncthreads();
    if (threadIdx.x == 0) {
      for (int w = 0; w < 8; ++w) b = sh.cand[w] > b ? sh.cand[w] : b;
      const int tok = static_cast<int>(~static_cast<uint32_t>(b));
      // no candidate (every score NaN): token -1 and no advance, as for a wait that gave up
      const bool ok = tok >= 0 && tok < a.vocab;
      a.tokens[0] = ok ? tok : -1;
      if (ok) advance_row(tok, a.ids, a.pos, a.len, a.slot, a.bt, a.bt_stride, a.history, a.max_position);
      a.rng[1] = st.stepc + 1;
    }
  }
  if (threadIdx.x == 0) __hip_atomic_store(a.epoch, ep + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace gr
