// Packed causal prefill attention on MFMA for the prompt-chunk tokens of a mixed step.
//
// "One forward per step", section "What changed": chunk positions stay packed and run the prefill
// kernel, decode positions get one query row per request. Here a chunk's tokens are cut into tiles
// of 16 consecutive queries of one request; one block handles one (tile, query head), and each of its
// waves a quarter of the tile's key blocks:
//   S^T[key][query] = K Q^T            v_mfma_f32_16x16x32 (K straight from the pool, Q from registers)
//   causal mask key_pos <= query_pos, online softmax per query (column)
//   O^T[dim][query] += V^T P^T          v_mfma_f32_16x16x16 (V^T fragments are 8-byte loads from the
//                                        dim-major V tile; the S^T accumulator layout is exactly the
//                                        P^T operand layout)
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

// Grid (tiles, nq), block 4 waves: block (tile, h) takes query head h of the tile, and its waves
// split the tile's key blocks (wave w: blocks w, w + 4, ...), each with its own online softmax;
// the four states merge in wave order through LDS at the end. A tile of the chunk's last queries
// sees the chunk's whole causal prefix, so one wave per (tile, head) would walk every key block in
// turn, one memory round trip each, on few waves per CU.
template <class T, int D>
__global__ __launch_bounds__(256) void k_attn_prefill(PrefillArgs a) {
  using S = typename T::S;
  constexpr int KS = D / 32;   // k-steps of the score MFMA
  constexpr int DT = D / 16;   // 16-dim output tiles
  __shared__ float wm[4][16], wl[4][16];
  __shared__ float wo[4][16][D];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int h = blockIdx.y;
  const int tile = blockIdx.x;
  const int req = a.tile_req[tile], q0 = a.tile_q0[tile];
  if (req < 0) return;         // padding tile (the tile list is padded to a fixed length); whole block
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
  const int nkb = maxpos / 16 + 1;
  // table entries of this wave's first 64 key blocks (lane j holds block wid + 4 j), fetched
  // before the loop
  const int bt_lane = wid + 4 * lane;
  const int bt_pre = (bt_lane < a.bt_stride) ? bt[bt_lane] : -1;
  auto pool_block = [&](int kb) -> int {   // kb is wave-uniform, one of this wave's blocks
    const int j = (kb - wid) / 4;
    int pb0;
    if (j < 64) pb0 = __builtin_amdgcn_readlane(bt_pre, j);
    else pb0 = (kb < a.bt_stride) ? bt[kb] : -1;
    return pb0 >= 0 ? pb0 : a.num_blocks - 1;
  };
  uint4 kf[KS];   // K fragment: key col, dims ks*32 + 8*grp .. + 8
  uint2 vf[DT];   // V^T fragment: dim t*16 + col, keys 4*grp .. + 4 (from the dim-major V tile)
  auto load_k = [&](int pb) {
    const S* kp = static_cast<const S*>(a.k_pool) + (static_cast<size_t>(pb) * a.nkv + g) * 16 * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kf[ks] = *reinterpret_cast<const uint4*>(kp + col * D + ks * 32 + 8 * grp);
  };
  auto load_v = [&](int pb) {
    const S* vp = static_cast<const S*>(a.v_pool) + (static_cast<size_t>(pb) * a.nkv + g) * 16 * D;
#pragma unroll
    for (int t = 0; t < DT; ++t) vf[t] = *reinterpret_cast<const uint2*>(vp + (t * 16 + col) * 16 + 4 * grp);
  };
  if (wid < nkb) {
    const int pb = pool_block(wid);
    load_k(pb);
    load_v(pb);
  }
  // software-pipelined: block kb + 4's K is requested once block kb's score product has issued,
  // its V once the value product has
  for (int kb = wid; kb < nkb; kb += 4) {
    const bool more = kb + 4 < nkb;
    const int next = pool_block(more ? kb + 4 : kb);
    f32x4_t s = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) s = mfma16x16x32<T>(kf[ks], qf[ks], s);
    if (more) load_k(next);
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
    if (kb * 16 + 15 > maxpos) {
      // keys past the tile's last query are not written yet: zero them so 0 * garbage cannot be NaN
      const int k0 = kb * 16 + 4 * grp;
      const uint32_t m0 = (k0 <= maxpos ? 0xffffu : 0u) | (k0 + 1 <= maxpos ? 0xffff0000u : 0u);
      const uint32_t m1 = (k0 + 2 <= maxpos ? 0xffffu : 0u) | (k0 + 3 <= maxpos ? 0xffff0000u : 0u);
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        vf[t].x &= m0;
        vf[t].y &= m1;
      }
    }
#pragma unroll
    for (int t = 0; t < DT; ++t) acc[t] = mfma16x16x16<T>(vf[t], pt, acc[t]);
    if (more) load_v(next);
  }
  // the four waves' states of each query (a wave without keys for a query has m = -inf), merged in
  // wave order; key 0 is visible to every query, so wave 0's state is never empty
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) wo[wid][col][t * 16 + 4 * grp + i] = acc[t][i];
  if (grp == 0) {
    wm[wid][col] = m;
    wl[wid][col] = lsum;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < cnt * D; e += 256) {
    const int qc = e / D, dd = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, wm[w][qc]);
    float Ls = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = (wm[w][qc] == -INFINITY) ? 0.f : __expf(wm[w][qc] - M);
      Ls += wl[w][qc] * f;
      O += wo[w][qc][dd] * f;
    }
    S* o = static_cast<S*>(a.out) + (static_cast<size_t>(q0 + qc) * a.nq + h) * D;
    o[dd] = T::from_f(O / Ls);
  }
}

}  // namespace gr
