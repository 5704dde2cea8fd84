// Mixture-of-experts MLP layer with no host reads: expert grouping and grouped GEMMs.
//
// "Removing overhead: fusion, graphs and async scheduling", section "A MoE layer that never asks
// the host": the N * k (token, slot) assignments are grouped by expert, each group padded to a
// multiple of BLOCK_M rows, with shapes that depend on N, k, E and BLOCK_M only; then one launch
// per projection multiplies each BLOCK_M-row block by its expert's weights, padding rows masked.
//
//   k_moe_align   the grouping (sorted_ids, block_expert, num_padded), one block of 16 waves.
//                 The lanes of a wave that hold the same expert are found with one ballot per id
//                 bit; the group's lowest lane counts the group (one LDS atomic per expert per
//                 wave). A block scan gives the padded group starts. Then, 1,024 assignments at a
//                 time, an assignment's place = its group's start + the earlier assignments of its
//                 expert (earlier chunks, earlier waves of this chunk, earlier lanes of its wave),
//                 so the order inside a group is assignment order, as a stable sort gives.
//   k_moe_gemm    one grouped GEMM on the matrix cores. Block = (16-row group block, tile of
//                 output columns): the expert's weight rows are the 16-row MFMA operand, the
//                 block's 16 gathered rows the other one, and the four waves take interleaved
//                 32-wide K steps whose partial tiles are summed in wave order through LDS. When
//                 experts average 32 rows or more, one workgroup takes up to 4 group blocks of an
//                 expert, so a weight fragment feeds up to 4 products. The hardware deals
//                 workgroups to the 8 XCDs in turn: XCD x takes group blocks x, x + 8, ... and all
//                 output tiles of each, so a block's input rows stay in one L2 and the live
//                 blocks spread evenly over the XCDs.
//                 GATE_UP: rows from the token (assignment / k); each tile is 8 gate rows and
//                 the matching 8 up rows, and the epilogue writes SiLU(gate) * up in the dtype
//                 (the page's SiLU-and-mul, fused), one row per grouped row, so the next GEMM
//                 reads each block's rows contiguously. DOWN: rows in grouped order, scaled by
//                 the router weight, written as fp32 rows in assignment order.
//   k_moe_sum     out[t] = the sum of token t's k rows in slot order (ids outside [0, E) add
//                 nothing), rounded to the dtype.
//
// Expert ids outside [0, E) belong to no group. Blocks whose first row lies at or past
// num_padded exit at once, so the grid is sized for the worst case.
#pragma once
#include "common.h"
#include "gemm.h"

namespace gr {

constexpr int kMoeBlockM = 16;        // rows per group block of the grouped GEMMs
constexpr int kMoeMaxExperts = 1024;
constexpr int kMoeAlignThreads = 1024;
constexpr int kXcds = 8;              // XCDs of an MI355X, each with its own L2

// lanes of this wave holding the same valid expert as this lane (ok: this lane's id is valid);
// one ballot per bit of the id
__device__ inline unsigned long long same_expert_lanes(int e, bool ok, int nbits) {
  unsigned long long peers = __ballot(ok);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = ok && ((e >> b) & 1);
    const unsigned long long m = __ballot(bit);
    peers &= bit ? m : ~m;
  }
  return peers;
}

__global__ __launch_bounds__(kMoeAlignThreads) void k_moe_align(const int* __restrict__ ids, int total, int E, int bm,
                                                                int m_max, int* __restrict__ sorted_ids,
                                                                int* __restrict__ block_expert, int* __restrict__ num_padded,
                                                                int* __restrict__ block_rank) {
  constexpr int NW = kMoeAlignThreads / 64;
  __shared__ int cnt[kMoeMaxExperts], pstart[kMoeMaxExperts];
  __shared__ int wcnt[NW][kMoeMaxExperts];   // per chunk: assignments of each expert in each wave
  __shared__ int wsum[NW];
  const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
  const unsigned long long lt = (1ull << lane) - 1ull;
  int nbits = 1;
  while ((1 << nbits) < E) ++nbits;
  for (int e = t; e < E; e += kMoeAlignThreads) cnt[e] = 0;
  __syncthreads();
  // counts: the lowest lane of each same-expert group of a wave adds the group's size
  for (int c0 = 0; c0 < total; c0 += kMoeAlignThreads) {
    const int i = c0 + t;
    const int e = i < total ? ids[i] : -1;
    const bool ok = e >= 0 && e < E;
    const unsigned long long peers = same_expert_lanes(e, ok, nbits);
    if (ok && (peers & lt) == 0ull) atomicAdd(&cnt[e], __popcll(peers));
  }
  __syncthreads();
  // exclusive scan of the padded counts (E <= kMoeAlignThreads: one expert per thread)
  const int c = t < E ? cnt[t] : 0;
  const int pad = (c + bm - 1) / bm * bm;
  int incl = pad;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wsum[wid] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wid; ++w) before += wsum[w];
  const int start = before + incl - pad;
  if (t < E) pstart[t] = start;
  if (t == kMoeAlignThreads - 1) num_padded[0] = before + incl;   // the grand total
  __syncthreads();
  const int npad = pstart[E - 1] + (cnt[E - 1] + bm - 1) / bm * bm;
  // padding rows of each group and the blocks each group owns
  if (t < E) {
    for (int r = start + c; r < start + pad; ++r) sorted_ids[r] = total;
    for (int b = start / bm; b < (start + pad) / bm; ++b) {
      block_expert[b] = t;
      if (block_rank) block_rank[b] = b - start / bm;
    }
  }
  for (int r = npad + t; r < m_max; r += kMoeAlignThreads) sorted_ids[r] = total;
  for (int b = npad / bm + t; b < m_max / bm; b += kMoeAlignThreads) {
    block_expert[b] = E - 1;
    if (block_rank) block_rank[b] = 0;
  }
  // places, one chunk of kMoeAlignThreads assignments at a time: place = group start + earlier
  // assignments of the expert in earlier chunks (run, kept by the expert's thread in pstart) +
  // in earlier waves of this chunk + in earlier lanes of this wave
  for (int c0 = 0; c0 < total; c0 += kMoeAlignThreads) {
    for (int e = lane; e < E; e += 64) wcnt[wid][e] = 0;
    __syncthreads();
    const int i = c0 + t;
    const int e = i < total ? ids[i] : -1;
    const bool ok = e >= 0 && e < E;
    const unsigned long long peers = same_expert_lanes(e, ok, nbits);
    if (ok && (peers & lt) == 0ull) wcnt[wid][e] = __popcll(peers);
    __syncthreads();
    if (t < E) {   // expert t: exclusive prefix over the waves, from its running place
      int run = pstart[t];
      for (int w = 0; w < NW; ++w) {
        const int v = wcnt[w][t];
        wcnt[w][t] = run;
        run += v;
      }
      pstart[t] = run;
    }
    __syncthreads();
    if (ok) sorted_ids[wcnt[wid][e] + __popcll(peers & lt)] = i;
    __syncthreads();
  }
}

struct MoeGemmArgs {
  const void* W;              // [E][wrows][K] expert weights
  const void* A;              // GATE_UP: token rows [N][K]; DOWN: activation rows [m_max][K] (grouped order)
  const int* sorted_ids;      // [m_max]
  const int* block_expert;    // [m_max / 16]
  const int* num_padded;      // [1]
  const int* block_rank;      // [m_max / 16] rank of each group block inside its expert's group (MB > 1)
  const float* weights;       // DOWN: router weight per assignment [N * k]
  void* out;                  // GATE_UP: activation rows (dtype) [m_max][ncols] in grouped order;
                              // DOWN: fp32 rows [N * k][ncols] in assignment order
  int ncols;                  // output columns: the expert width I (GATE_UP) or the hidden size D (DOWN)
  int K;                      // reduction length, a multiple of 32
  int total, top_k;
  int ntiles;                 // output tiles; gridDim.x = (m_max / 16 rounded up to a multiple of 8) * ntiles
};

// RT tiles per block; GATE_UP tiles are 8 output columns (8 gate + 8 up weight rows), DOWN tiles 16.
// MB > 1: the workgroup of a group block whose rank inside its expert's group is a multiple of MB
// also takes the next MB - 1 group blocks of that group (the others exit), so each weight fragment
// feeds up to MB products.
template <class T, bool GATE_UP, int RT, int UN, int MB>
__global__ __launch_bounds__(256) void k_moe_gemm(MoeGemmArgs a) {
  using S = typename T::S;
  __shared__ f32x4_t part[4][MB][64];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  // workgroup b runs on XCD b % 8 as the (b / 8)-th of that XCD's share: XCD x takes the group
  // blocks x, x + 8, ... and, for each, every tile in turn
  const int xcd = blockIdx.x % kXcds, slot = static_cast<int>(blockIdx.x) / kXcds;
  const int mb = xcd + kXcds * (slot / a.ntiles), nt = slot % a.ntiles;
  const int npad = a.num_padded[0];
  if (mb * kMoeBlockM >= npad) return;
  int cnt = 1;   // group blocks of this workgroup
  if constexpr (MB > 1) {
    const int rank = a.block_rank[mb];
    if (rank % MB) return;
    for (int i = 1; i < MB; ++i) {
      if ((mb + i) * kMoeBlockM >= npad || a.block_rank[mb + i] != rank + i) break;
      cnt = i + 1;
    }
  }
  const int K = a.K;
  const int wrows = GATE_UP ? 2 * a.ncols : a.ncols;
  const int expert = a.block_expert[mb];
  const S* W = static_cast<const S*>(a.W) + static_cast<size_t>(expert) * wrows * K;
  const uint4 zero4 = make_uint4(0, 0, 0, 0);
  const int koff = 8 * (lane >> 4);
  // this lane's weight row in each tile (clamped in bounds; rows past the end are zeroed)
  const S* wp[RT];
  bool wok[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    int wrow;
    if (GATE_UP) {
      const int j = (nt * RT + r) * 8 + (lane & 7);
      wrow = ((lane & 15) < 8) ? j : a.ncols + j;
      wok[r] = j < a.ncols;
    } else {
      wrow = (nt * RT + r) * 16 + (lane & 15);
      wok[r] = wrow < a.ncols;
    }
    wp[r] = W + static_cast<size_t>(min(wrow, wrows - 1)) * K + koff;
  }
  // this lane's gathered row in each group block (row lane % 16); padding rows and group blocks
  // past cnt read row 0, zeroed
  // (GATE_UP: the token's row; DOWN: the activation row, stored in grouped order)
  int asg[MB];
  bool aok[MB];
  const S* ap[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int grow = (mb + i) * kMoeBlockM + (lane & 15);
    asg[i] = i < cnt ? a.sorted_ids[grow] : a.total;
    aok[i] = asg[i] < a.total;
    const int src = aok[i] ? (GATE_UP ? asg[i] / a.top_k : grow) : 0;
    ap[i] = static_cast<const S*>(a.A) + static_cast<size_t>(src) * K + koff;
  }

  f32x4_t acc[RT][MB];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int i = 0; i < MB; ++i) acc[r][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int ksteps = K / 32;
  int ks = wid;
  for (; ks + 4 * (UN - 1) < ksteps; ks += 4 * UN) {
    uint4 wv[UN][RT], av[UN][MB];
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int k = (ks + 4 * u) * 32;
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        wv[u][r] = *reinterpret_cast<const uint4*>(wp[r] + k);
        if (!wok[r]) wv[u][r] = zero4;
      }
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        av[u][i] = zero4;
        if (i < cnt) av[u][i] = *reinterpret_cast<const uint4*>(ap[i] + k);
        if (!aok[i]) av[u][i] = zero4;
      }
    }
#pragma unroll
    for (int u = 0; u < UN; ++u)
#pragma unroll
      for (int i = 0; i < MB; ++i)
        if (i < cnt)
#pragma unroll
          for (int r = 0; r < RT; ++r) acc[r][i] = mfma16x16x32<T>(wv[u][r], av[u][i], acc[r][i]);
  }
  for (; ks < ksteps; ks += 4) {
    const int k = ks * 32;
    uint4 wv[RT], av[MB];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      wv[r] = *reinterpret_cast<const uint4*>(wp[r] + k);
      if (!wok[r]) wv[r] = zero4;
    }
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      av[i] = zero4;
      if (i < cnt) av[i] = *reinterpret_cast<const uint4*>(ap[i] + k);
      if (!aok[i]) av[i] = zero4;
    }
#pragma unroll
    for (int i = 0; i < MB; ++i)
      if (i < cnt)
#pragma unroll
        for (int r = 0; r < RT; ++r) acc[r][i] = mfma16x16x32<T>(wv[r], av[i], acc[r][i]);
  }
  // tile by tile, the four waves' partial sums meet in LDS and wave r keeps tile r's sum (RT <= 4)
  f32x4_t sum[MB];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
#pragma unroll
    for (int i = 0; i < MB; ++i) part[wid][i][lane] = acc[r][i];
    __syncthreads();
    if (wid == r) {
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        sum[i] = part[0][i][lane];
#pragma unroll
        for (int w = 1; w < 4; ++w) sum[i] += part[w][i][lane];
      }
    }
    __syncthreads();
  }
  const int r = wid;
  if (r >= RT) return;
  const int cb = 4 * (lane >> 4);     // first of the 4 weight rows this lane holds
  // the MFMA result holds weight rows (4 per lane) x group-block rows (lane % 16: one assignment)
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    if (i >= cnt) break;
    if (GATE_UP) {
      // lanes 0..31 hold gate rows 0..7 of the tile, lanes 32..63 the matching up rows
      f32x4_t up;
#pragma unroll
      for (int q = 0; q < 4; ++q) up[q] = __shfl(sum[i][q], lane + 32, 64);
      if (lane < 32 && aok[i]) {
        S* out = static_cast<S*>(a.out) + static_cast<size_t>((mb + i) * kMoeBlockM + (lane & 15)) * a.ncols;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j = (nt * RT + r) * 8 + cb + q;
          if (j < a.ncols) out[j] = T::from_f(silu(sum[i][q]) * up[q]);
        }
      }
    } else if (aok[i]) {
      const float wgt = a.weights[asg[i]];
      float* out = static_cast<float*>(a.out) + static_cast<size_t>(asg[i]) * a.ncols;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = (nt * RT + r) * 16 + cb + q;
        if (n < a.ncols) out[n] = sum[i][q] * wgt;
      }
    }
  }
}

// out[t][c] = sum over slots j of rows[t * k + j][c] (valid experts only), in slot order; four
// columns per thread, grid (tokens, D / 1024 rounded up), every slot's load issued at once.
template <class T>
__global__ __launch_bounds__(256) void k_moe_sum(const float* __restrict__ rows, const int* __restrict__ ids, int k,
                                                 int E, int D, void* __restrict__ out) {
  using S = typename T::S;
  const int tk = blockIdx.x;
  const int c = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (c >= D) return;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  constexpr int KU = 8;
  for (int j0 = 0; j0 < k; j0 += KU) {
    float4 v[KU];
    bool ok[KU];
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int j = min(j0 + u, k - 1);
      const int e = ids[tk * k + j];
      ok[u] = j0 + u < k && e >= 0 && e < E;
      v[u] = *reinterpret_cast<const float4*>(rows + (static_cast<size_t>(tk) * k + j) * D + c);
    }
#pragma unroll
    for (int u = 0; u < KU; ++u)
      if (ok[u]) {
        s.x += v[u].x;
        s.y += v[u].y;
        s.z += v[u].z;
        s.w += v[u].w;
      }
  }
  S* o = static_cast<S*>(out) + static_cast<size_t>(tk) * D + c;
  o[0] = T::from_f(s.x);
  o[1] = T::from_f(s.y);
  o[2] = T::from_f(s.z);
  o[3] = T::from_f(s.w);
}

}  // namespace gr
