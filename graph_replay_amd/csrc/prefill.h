// Packed causal prefill attention on MFMA for the prompt-chunk tokens of a mixed step.
//
// "One forward per step", section "What changed": chunk positions stay packed and run the prefill
// kernel, decode positions get one query row per request. Here a chunk's tokens are cut into tiles
// of 16 consecutive queries of one request; one wave handles one (tile, query head):
//   S^T[key][query] = K Q^T            v_mfma_f32_16x16x32 (K straight from the pool, Q from registers)
//   causal mask key_pos <= query_pos, online softmax per query (column)
//   O^T[dim][query] += V^T P^T          v_mfma_f32_16x16x16 (V^T fragments from a per-wave LDS tile;
//                                        the S^T accumulator layout is exactly the P^T operand layout)
// MFMA lane layout (16x16 tiles): operand A lane l holds row l % 16 and the k slots of lane group
// l / 16, operand B holds column l % 16 and the same k slots, and the accumulator holds rows
// 4 * (l / 16) + i (i = 0..3) of column l % 16.
#pragma once
#include "common.h"
#include "gemm.h"

namespace gr {

struct PrefillArgs {
  int nq, nkv;
  const float* q;            // [tokens][nq][D] fp32, RMSNorm'd + RoPE'd queries
  const void* k_pool;
  const void* v_pool;
  const int* block_table;    // [reqs][bt_stride]
  int bt_stride;
  const int* tile_req;       // [tiles] request of the tile
  const int* tile_q0;        // [tiles] first packed token of the tile
  const int* qsl;            // [reqs + 1] token offsets of the requests
  const int* pos;            // [tokens] absolute positions
  int num_blocks;
  float scale;
  void* out;                 // [tokens][nq * D] model dtype
};

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));

template <class T>
__device__ inline f32x4_t mfma16x16x16(const uint2& a, const uint2& b, f32x4_t c) {
  if constexpr (__is_same(T, BF16)) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a), __builtin_bit_cast(i16x4_t, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a), __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
  }
}

template <class T>
__device__ inline uint32_t pack2(float x, float y) {
  using S = typename T::S;
  S a = T::from_f(x), b = T::from_f(y);
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) | (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}

// Grid (tiles, ceil(nq / 4)), block 4 waves; wave w takes query head blockIdx.y * 4 + w.
template <class T, int D>
__global__ __launch_bounds__(256) void k_attn_prefill(PrefillArgs a) {
  using S = typename T::S;
  constexpr int KS = D / 32;   // k-steps of the score MFMA
  constexpr int DT = D / 16;   // 16-dim output tiles
  __shared__ __align__(16) S vt[4][16 * D];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int h = blockIdx.y * 4 + wid;
  if (h >= a.nq) return;       // waves never synchronise with each other
  const int tile = blockIdx.x;
  const int req = a.tile_req[tile], q0 = a.tile_q0[tile];
  const int cnt = min(16, a.qsl[req + 1] - q0);
  const int g = h / (a.nq / a.nkv);
  const int col = lane & 15, grp = lane >> 4;
  const int qi = min(col, cnt - 1);            // queries past the tile end duplicate its last one
  const int qpos = a.pos[q0 + qi];
  const int maxpos = a.pos[q0 + cnt - 1];      // positions rise within a chunk
  const int* bt = a.block_table + static_cast<size_t>(req) * a.bt_stride;

  // Q^T fragments: column = this lane's query, k slots = dims ks*32 + 8*grp .. + 8
  uint4 qf[KS];
  const float* qrow = a.q + (static_cast<size_t>(q0 + qi) * a.nq + h) * D;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const float* src = qrow + ks * 32 + 8 * grp;
    qf[ks] = make_uint4(pack2<T>(src[0] * a.scale, src[1] * a.scale), pack2<T>(src[2] * a.scale, src[3] * a.scale),
                        pack2<T>(src[4] * a.scale, src[5] * a.scale), pack2<T>(src[6] * a.scale, src[7] * a.scale));
  }

  f32x4_t acc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;
  S* vs = vt[wid];
  const int nkb = maxpos / 16 + 1;
  for (int kb = 0; kb < nkb; ++kb) {
    const int pb0 = (kb < a.bt_stride) ? bt[kb] : -1;
    const int pb = pb0 >= 0 ? pb0 : a.num_blocks - 1;
    const size_t tileoff = (static_cast<size_t>(pb) * a.nkv + g) * 16 * D;
    const S* kp = static_cast<const S*>(a.k_pool) + tileoff;
    const S* vp = static_cast<const S*>(a.v_pool) + tileoff;
    uint4 kf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kf[ks] = *reinterpret_cast<const uint4*>(kp + col * D + ks * 32 + 8 * grp);
    // stage the V tile (16 keys x D) in this wave's LDS
    constexpr int VPL = 16 * D * static_cast<int>(sizeof(S)) / 16 / 64;   // 16-byte vectors per lane
    uint4 vv[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) vv[i] = reinterpret_cast<const uint4*>(vp)[lane + 64 * i];
    f32x4_t s = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) s = mfma16x16x32<T>(kf[ks], qf[ks], s);
    // causal mask; this lane holds keys kb*16 + 4*grp + i of query `col`
    float bm = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kpos = kb * 16 + 4 * grp + i;
      s[i] = (kpos <= qpos) ? s[i] : -INFINITY;
      bm = fmaxf(bm, s[i]);
    }
    bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
    bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
    const float mn = fmaxf(m, bm);
    const float corr = (m == -INFINITY) ? 0.f : __expf(m - mn);
    float p[4], ps = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = (s[i] == -INFINITY) ? 0.f : __expf(s[i] - mn);
      ps += p[i];
    }
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    lsum = lsum * corr + ps;
    m = mn;
#pragma unroll
    for (int t = 0; t < DT; ++t) acc[t] *= corr;
    const uint2 pt = make_uint2(pack2<T>(p[0], p[1]), pack2<T>(p[2], p[3]));
    // keys past the tile's last query are not written yet: zero them so 0 * garbage cannot be NaN
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int key = (lane + 64 * i) * 16 / static_cast<int>(sizeof(S)) / D;   // key of this 16-byte vector
      reinterpret_cast<uint4*>(vs)[lane + 64 * i] = (kb * 16 + key <= maxpos) ? vv[i] : make_uint4(0, 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      // V^T fragment: row = dim t*16 + col, k slots = keys 4*grp .. 4*grp+3
      const int dim = t * 16 + col;
      const uint16_t e0 = __builtin_bit_cast(uint16_t, vs[(4 * grp + 0) * D + dim]);
      const uint16_t e1 = __builtin_bit_cast(uint16_t, vs[(4 * grp + 1) * D + dim]);
      const uint16_t e2 = __builtin_bit_cast(uint16_t, vs[(4 * grp + 2) * D + dim]);
      const uint16_t e3 = __builtin_bit_cast(uint16_t, vs[(4 * grp + 3) * D + dim]);
      const uint2 va = make_uint2(e0 | (static_cast<uint32_t>(e1) << 16), e2 | (static_cast<uint32_t>(e3) << 16));
      acc[t] = mfma16x16x16<T>(va, pt, acc[t]);
    }
    __builtin_amdgcn_wave_barrier();
  }
  if (col < cnt) {
    S* o = static_cast<S*>(a.out) + (static_cast<size_t>(q0 + col) * a.nq + h) * D;
    const float inv = 1.0f / lsum;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[t * 16 + 4 * grp + i] = T::from_f(acc[t][i] * inv);
  }
}

}  // namespace gr
