// Device-side sampling and the in-place advance of the decode state.
//
// Sampling follows "Fast decode: syncs, CUDA graphs and compilation", section "Sampling without the
// CPU": temperature 0 takes the argmax of the logits; otherwise u is clamped to [1e-10, 1],
// g = -log(-log u) and the token is argmax(z / T + g), an exact draw from softmax(z / T). Ties go
// to the lowest index. Uniforms come from a caller buffer or from Philox-4x32-10 (Salmon et al.,
// "Parallel random numbers: as easy as 1, 2, 3", SC'11) with key (seed low, seed high) and counter
// (column / 4, row, step low, step high); word j of a call is column 4 * (column / 4) + j and
// u = (word >> 8) * 2^-24.
//
// The advance follows the same page, section "The fast decoder": the sampled token becomes the next
// input, the position and the key count move by one, and the output is recorded at the input's
// position, all on the device, so nothing waits for the host.
#pragma once
#include "common.h"

namespace gr {

__device__ inline void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    // each 32 x 32 -> 64-bit product as one 64-bit multiply (one v_mad_u64_u32 instead of a
    // separate low and high multiply)
    const uint64_t p0 = static_cast<uint64_t>(0xD2511F53u) * c[0];
    const uint64_t p1 = static_cast<uint64_t>(0xCD9E8D57u) * c[2];
    const uint32_t lo0 = static_cast<uint32_t>(p0), hi0 = static_cast<uint32_t>(p0 >> 32);
    const uint32_t lo1 = static_cast<uint32_t>(p1), hi1 = static_cast<uint32_t>(p1 >> 32);
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
}

// The Gumbel-max score of a temperature-scaled logit zd = z / T (T > 0) with uniform u. The two
// natural logs use the hardware log2 (v_log_f32, about one ulp) scaled by ln 2: the full-precision
// library log costs some twenty more instructions each, and the sampler spends them on every logit
// of every sampled row. Every sampler here (k_sample, the fused LM heads) scores with this function,
// so their tokens agree bit for bit.
__device__ inline float gumbel_score(float zd, float u) {
  const float uu = fminf(fmaxf(u, 1e-10f), 1.0f);
  return zd - __logf(-__logf(uu));
}

// The uniform of (row, column) under the counter scheme above, from one Philox call.
__device__ inline float philox_uniform(uint64_t seed, uint64_t step, int row, int col) {
  uint32_t w[4] = {static_cast<uint32_t>(col >> 2), static_cast<uint32_t>(row), static_cast<uint32_t>(step),
                   static_cast<uint32_t>(step >> 32)};
  philox4x32_10(w, static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32));
  const int j = col & 3;
  const uint32_t x = j == 0 ? w[0] : j == 1 ? w[1] : j == 2 ? w[2] : w[3];
  return static_cast<float>(x >> 8) * 5.9604644775390625e-08f;
}

// The in-place advance of one decode row whose token is tok: the token is recorded at the input's
// position and becomes the next input, and the position and key count move by one; a row out of
// positions (hist_ld) or of reserved blocks turns into a padding row. Padding rows (len 0) stay.
__device__ inline void advance_row(int tok, int* ids, int* pos, int* lens, int* slots, const int* bt_row,
                                   int bt_stride, int* hist_row, int hist_ld) {
  const int len = *lens;
  if (len <= 0) return;
  const int p = *pos;
  if (hist_row && p < hist_ld) hist_row[p] = tok;
  const int np = p + 1;
  const int blk = np / 16;
  const int entry = (blk < bt_stride) ? bt_row[blk] : -1;
  if (np >= hist_ld || entry < 0) {
    *ids = 0;
    *pos = 0;
    *lens = 0;
    *slots = -1;
  } else {
    *ids = tok;
    *pos = np;
    *lens = len + 1;
    *slots = entry * 16 + np % 16;
  }
}

// ------------------------------------------------------------------------------------------------
// Top-k / top-p filters before the Gumbel-max argmax (same page and section: the filters run before
// the argmax and set filtered logits to -inf; a fixed k keeps shapes static, and top-p is a sort and
// a mask). Readings: both act only at T > 0, on z = logit / T in fp32; top-k keeps every z >= the
// k-th largest (k <= 0 or k >= V: off); top-p acts on the softmax of the top-k-kept z, in the order
// (z descending, index ascending), and keeps a token while the mass before it is < p (p >= 1: off).
//
// k_sample_filter writes per row a pair (x, y): token i is kept iff key_i > x or (key_i == x and
// i < y), key being an order-preserving 32-bit key of z. One block of 1024 threads per row:
//   * a key range known to hold the cut is split into 2048 bins (counts for top-k, masses for
//     top-p), the bin holding the cut is found by a scan from the top bin down, and the range
//     shrinks to that bin, until the bin holds at most 2048 tokens or a single key value;
//   * the bin's tokens are gathered into LDS and sorted by (key desc, index asc), which gives the
//     cut exactly; a single key value with more tokens than that (a run of exact ties) is cut by
//     a scan in index order.
// Masses are exp(z - zmax) in fixed point (units of 2^-31, truncated) summed as 64-bit integers, so
// every sum is exact and independent of thread order: the filter is deterministic. Top-p looks at
// tokens within 30 of zmax (their mass is all but < 2e-8 of the total): when p asks for more than
// that window holds, the whole top-k set is kept.
__device__ inline uint32_t fkey(float z) {
  const uint32_t u = (z == 0.f) ? 0u : __float_as_uint(z);   // -0 and +0 share a key
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ inline float fkey_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
// The sampler's order (score descending, then index ascending) as one unsigned 64-bit key: the
// order-preserving key of the score above the complemented index. A NaN score gets key 0, below
// every real candidate, as it never wins the sampler's comparisons.
__device__ inline unsigned long long score_key(float sc, int idx) {
  if (sc != sc) return 0ull;
  return (static_cast<unsigned long long>(fkey(sc)) << 32) | static_cast<uint32_t>(~idx);
}
// the largest 64-bit value over the wave, in every lane
__device__ inline unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), o, 64);
    const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), o, 64);
    const unsigned long long w = (static_cast<unsigned long long>(hi) << 32) | lo;
    v = w > v ? w : v;
  }
  return v;
}
__device__ inline unsigned long long qmass(float z, float zmax) {
  return static_cast<unsigned long long>(static_cast<uint32_t>(__expf(z - zmax) * 2147483648.0f));
}

struct FilterArgs {
  const float* logits;
  int ld, vocab;
  const float* temperature;           // [rows] or nullptr (greedy: nothing filtered)
  const int* top_k;                   // [rows] or nullptr
  const float* top_p;                 // [rows] or nullptr
  const int* n_rows;                  // device row count (nullptr: gridDim.x); rows past it are idle
  uint2* filt;                        // [rows] out: (x, y)
};

constexpr int kFilterThreads = 1024;

__device__ inline unsigned long long shfl_up_u64(unsigned long long v, int d) {
  const unsigned lo = __shfl_up(static_cast<unsigned>(v), d, 64);
  const unsigned hi = __shfl_up(static_cast<unsigned>(v >> 32), d, 64);
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}

// exclusive scan over the block in thread order (all threads call it); wtot: 16 entries of LDS
__device__ inline unsigned long long block_excl_scan(unsigned long long v, unsigned long long* wtot,
                                                     unsigned long long* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  unsigned long long inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const unsigned long long o = shfl_up_u64(inc, d);
    if (lane >= d) inc += o;
  }
  __syncthreads();
  if (lane == 63) wtot[wid] = inc;
  __syncthreads();
  unsigned long long base = 0, all = 0;
  for (int w = 0; w < nw; ++w) {
    if (w < wid) base += wtot[w];
    all += wtot[w];
  }
  *total = all;
  return base + inc - v;
}

static __global__ __launch_bounds__(kFilterThreads) void k_sample_filter(FilterArgs a) {
  constexpr int NB = 2048, CAP = 2048, NT = kFilterThreads;
  __shared__ unsigned hcnt[NB];
  __shared__ unsigned long long hmass[NB];
  __shared__ uint32_t ckey[CAP];
  __shared__ int cidx[CAP];
  __shared__ unsigned long long wtot[NT / 64];
  __shared__ float wred[NT / 64];
  __shared__ int s_bin, s_n, s_idx;
  __shared__ unsigned long long s_above;
  const int row = blockIdx.x, t = threadIdx.x, lane = t & 63, wid = t >> 6;
  if (a.n_rows && row >= *a.n_rows) return;
  const int V = a.vocab;
  const float T = a.temperature ? a.temperature[row] : 0.f;
  const int k = a.top_k ? a.top_k[row] : 0;
  const float p = a.top_p ? a.top_p[row] : 1.f;
  const bool use_k = T > 0.f && k > 0 && k < V;
  const bool use_p = T > 0.f && p < 1.f;
  if (!use_k && !use_p) {
    if (t == 0) a.filt[row] = make_uint2(0u, 0x7fffffffu);
    return;
  }
  const float* lg = a.logits + static_cast<size_t>(row) * a.ld;

  // zmax and zmin (block reductions in a fixed order)
  float zmx = -INFINITY, zmn = INFINITY;
  for (int i = t; i < V; i += NT) {
    const float z = lg[i] / T;
    zmx = fmaxf(zmx, z);
    zmn = fminf(zmn, z);
  }
  zmx = wave_max(zmx);
  zmn = -wave_max(-zmn);
  if (lane == 0) wred[wid] = zmx;
  __syncthreads();
  float zmax = -INFINITY;
  for (int w = 0; w < NT / 64; ++w) zmax = fmaxf(zmax, wred[w]);
  __syncthreads();
  if (lane == 0) wred[wid] = zmn;
  __syncthreads();
  float zmin = INFINITY;
  for (int w = 0; w < NT / 64; ++w) zmin = fminf(zmin, wred[w]);
  __syncthreads();

  // Find the cut in [lo, hi] (keys >= kmin only): by count (target = k, above = count of kept keys
  // above hi) or by mass (target = p * Z). Returns (x, y) for the kept set, or found = false when
  // the range holds too little (mass phase: the cut is below the window).
  auto select = [&](bool by_mass, uint32_t lo, uint32_t hi, uint32_t kmin, double target,
                    unsigned long long above, uint2* out) -> bool {
    for (;;) {
      for (int i = t; i < NB; i += NT) { hcnt[i] = 0u; hmass[i] = 0ull; }
      __syncthreads();
      const unsigned long long W = static_cast<unsigned long long>(hi) - lo + 1ull;
      for (int i = t; i < V; i += NT) {
        const float z = lg[i] / T;
        const uint32_t key = fkey(z);
        if (key < lo || key > hi || key < kmin) continue;
        const int bin = static_cast<int>((static_cast<unsigned long long>(key - lo) * NB) / W);
        atomicAdd(&hcnt[bin], 1u);
        if (by_mass) atomicAdd(&hmass[bin], qmass(z, zmax));
      }
      if (t == 0) s_bin = -1;
      __syncthreads();
      // descending bins: thread t holds bins NB-1-2t and NB-2-2t
      const int b0 = NB - 1 - 2 * t, b1 = b0 - 1;
      const unsigned long long v0 = by_mass ? hmass[b0] : hcnt[b0], v1 = by_mass ? hmass[b1] : hcnt[b1];
      unsigned long long tot;
      const unsigned long long ex = block_excl_scan(v0 + v1, wtot, &tot) + above;
      if (static_cast<double>(ex) < target && target <= static_cast<double>(ex + v0)) {
        s_bin = b0;
        s_above = ex;
      } else if (static_cast<double>(ex + v0) < target && target <= static_cast<double>(ex + v0 + v1)) {
        s_bin = b1;
        s_above = ex + v0;
      }
      __syncthreads();
      const int b = s_bin;
      if (b < 0) return false;
      above = s_above;
      const unsigned n = hcnt[b];
      const uint32_t nlo = lo + static_cast<uint32_t>((static_cast<unsigned long long>(b) * W + NB - 1) / NB);
      const uint32_t nhi = lo + static_cast<uint32_t>(((static_cast<unsigned long long>(b) + 1) * W + NB - 1) / NB) - 1u;
      __syncthreads();
      lo = nlo;
      hi = nhi;
      if (n <= CAP) {
        // gather the bin, sort by (key desc, index asc), cut exactly
        if (t == 0) s_n = 0;
        for (int i = t; i < CAP; i += NT) { ckey[i] = 0u; cidx[i] = 0x7fffffff; }
        __syncthreads();
        for (int i = t; i < V; i += NT) {
          const uint32_t key = fkey(lg[i] / T);
          if (key < lo || key > hi || key < kmin) continue;
          const int pos = atomicAdd(&s_n, 1);
          ckey[pos] = key;
          cidx[pos] = i;
        }
        __syncthreads();
        for (int size = 2; size <= CAP; size <<= 1) {
          for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int e = t; e < CAP / 2; e += NT) {
              const int i = 2 * e - (e & (stride - 1));
              const int j = i + stride;
              const bool desc = ((i & size) == 0);   // first half of each run: (key desc, idx asc)
              const uint32_t ki = ckey[i], kj = ckey[j];
              const int ii = cidx[i], ij = cidx[j];
              const bool i_first = ki > kj || (ki == kj && ii < ij);
              if (i_first != desc) {
                ckey[i] = kj; ckey[j] = ki;
                cidx[i] = ij; cidx[j] = ii;
              }
            }
            __syncthreads();
          }
        }
        if (!by_mass) {
          if (t == 0) *out = make_uint2(ckey[static_cast<int>(target - static_cast<double>(above)) - 1], 0x7fffffffu);
        } else {
          // two sorted entries per thread, in order
          unsigned long long m0 = 2 * t < static_cast<int>(n) ? qmass(fkey_value(ckey[2 * t]), zmax) : 0ull;
          unsigned long long m1 = 2 * t + 1 < static_cast<int>(n) ? qmass(fkey_value(ckey[2 * t + 1]), zmax) : 0ull;
          if (t == 0) s_idx = -1;
          __syncthreads();
          unsigned long long tt;
          const unsigned long long e0 = block_excl_scan(m0 + m1, wtot, &tt) + above;
          int jsel = -1;
          if (2 * t < static_cast<int>(n) && target <= static_cast<double>(e0 + m0) && static_cast<double>(e0) < target) jsel = 2 * t;
          else if (2 * t + 1 < static_cast<int>(n) && target <= static_cast<double>(e0 + m0 + m1) &&
                   static_cast<double>(e0 + m0) < target) jsel = 2 * t + 1;
          if (jsel >= 0) s_idx = jsel;
          __syncthreads();
          const int j = s_idx;
          // rounding can leave the cut just past the last entry: keep the whole bin then
          if (t == 0) *out = (j >= 0) ? make_uint2(ckey[j], static_cast<uint32_t>(cidx[j]) + 1u)
                                      : make_uint2(ckey[n - 1], static_cast<uint32_t>(cidx[n - 1]) + 1u);
        }
        __syncthreads();
        return true;
      }
      if (lo == hi) {
        // one key value held by more than CAP tokens: exact ties
        if (!by_mass) {
          if (t == 0) *out = make_uint2(lo, 0x7fffffffu);
          __syncthreads();
          return true;
        }
        const unsigned long long q = qmass(fkey_value(lo), zmax);
        const double need = (target - static_cast<double>(above)) / static_cast<double>(q > 0 ? q : 1ull);
        const long long c = static_cast<long long>(fmax(1.0, ceil(need)));   // ties to keep
        if (c >= static_cast<long long>(n)) {
          if (t == 0) *out = make_uint2(lo, 0x7fffffffu);
          __syncthreads();
          return true;
        }
        // the c-th tie in index order: contiguous chunks per thread, exclusive scan of the counts
        const int ch = (V + NT - 1) / NT, c0 = t * ch, c1 = min(V, c0 + ch);
        unsigned own = 0;
        for (int i = c0; i < c1; ++i) own += (fkey(lg[i] / T) == lo) ? 1u : 0u;
        unsigned long long tt;
        const unsigned long long ex = block_excl_scan(own, wtot, &tt);
        if (static_cast<long long>(ex) < c && c <= static_cast<long long>(ex + own)) {
          long long r = c - static_cast<long long>(ex);
          for (int i = c0; i < c1; ++i)
            if (fkey(lg[i] / T) == lo && --r == 0) {
              s_idx = i;
              break;
            }
        }
        __syncthreads();
        if (t == 0) *out = make_uint2(lo, static_cast<uint32_t>(s_idx) + 1u);
        __syncthreads();
        return true;
      }
    }
  };

  __shared__ uint2 s_out;
  uint32_t kthr = 0u;
  if (use_k) {
    select(false, fkey(zmin), fkey(zmax), 0u, static_cast<double>(k), 0ull, &s_out);
    __syncthreads();
    kthr = s_out.x;
  }
  if (!use_p) {
    if (t == 0) a.filt[row] = make_uint2(kthr, 0x7fffffffu);
    return;
  }
  // top-p over the top-k set: Z = total mass of keys >= kthr (window bins + the tail below it)
  const uint32_t wlo = max(kthr, fkey(zmax - 30.f));
  unsigned long long zt = 0;
  for (int i = t; i < V; i += NT) {
    const float z = lg[i] / T;
    if (fkey(z) >= kthr) zt += qmass(z, zmax);
  }
  unsigned long long Z;
  (void)block_excl_scan(zt, wtot, &Z);
  __syncthreads();
  const double target = static_cast<double>(p) * static_cast<double>(Z);
  const bool found = select(true, wlo, fkey(zmax), kthr, target, 0ull, &s_out);
  __syncthreads();
  if (t == 0) a.filt[row] = found ? s_out : make_uint2(kthr, 0x7fffffffu);
}

struct SampleArgs {
  const float* logits;
  int ld, vocab, chunk;               // chunk: columns per block (multiple of 1024)
  const float* temperature;           // [rows] or nullptr (greedy)
  const float* uniforms;              // [rows][ld] or nullptr (Philox)
  const uint64_t* rng;                // device {seed, step} (decode) or nullptr
  uint64_t seed, step;                // used when rng == nullptr
  float* part_val;                    // [rows][nchunks]
  int* part_idx;
  unsigned* row_cnt;                  // [rows], zero between launches (reset by the row's last block)
  unsigned* done_cnt;                 // [1], zero between launches (reset by the last row)
  const int* n_rows;                  // device row count (nullptr: gridDim.x); rows past it are idle
  const uint2* filt;                  // [rows] top-k / top-p cut from k_sample_filter, or nullptr
  int* tokens_out;                    // [rows]
  // decode advance (advance != 0)
  int advance;
  int* input_ids;
  int* positions;
  int* seq_lens;
  int* slots;
  const int* block_table;
  int bt_stride;
  int* history;                       // [rows][hist_ld] or nullptr
  int hist_ld;                        // max_position: positions at or past it end the row
  const int* halt;                    // nonzero *halt: the logits are invalid (token -1, no advance)
};

__device__ inline void best_merge(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}

__device__ inline void block_best(float& v, int& i, float* sv, int* si) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float v2 = __shfl_xor(v, o, 64);
    const int i2 = __shfl_xor(i, o, 64);
    best_merge(v, i, v2, i2);
  }
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if (lane == 0) { sv[wid] = v; si[wid] = i; }
  __syncthreads();
  v = sv[0];
  i = si[0];
  for (int w = 1; w < nw; ++w) best_merge(v, i, sv[w], si[w]);
}

// Grid (rows, nchunks), block 256. Each block scores its columns of one row; the last block of a
// row to finish merges the chunk winners (the order (value desc, index asc) is total, so the merge
// order cannot change the winner), writes the token and advances the row. The last row to finish
// moves the Philox step counter on: every block read it before it counted itself in.
static __global__ __launch_bounds__(256) void k_sample(SampleArgs a) {
  __shared__ float sv[4];
  __shared__ int si[4];
  __shared__ int last_flag;
  const int row = blockIdx.x, ch = blockIdx.y, nch = gridDim.y;
  // invalid logits (see halt): nothing advances, the Philox step counter included
  const bool halted = a.halt && ld_dev(a.halt) != 0;
  if (a.n_rows && row >= *a.n_rows) {
    // idle row: still counted in by one block, so the step counter and its reset stay exact
    if (ch == 0 && threadIdx.x == 0 && a.rng && arrive_last(a.done_cnt, gridDim.x) && !halted) {
      uint64_t* r = const_cast<uint64_t*>(a.rng);
      r[1] = r[1] + 1;
    }
    return;
  }
  const float T = a.temperature ? a.temperature[row] : 0.f;
  const uint64_t seed = a.rng ? a.rng[0] : a.seed;
  const uint64_t step = a.rng ? a.rng[1] : a.step;
  const float* z = a.logits + static_cast<size_t>(row) * a.ld;
  const int c0 = ch * a.chunk, c1 = min(a.vocab, c0 + a.chunk);
  const uint2 cut = a.filt ? a.filt[row] : make_uint2(0u, 0x7fffffffu);   // keep all when absent
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int c = c0 + 4 * threadIdx.x; c < c1; c += 4 * blockDim.x) {
    float zz[4], u[4] = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) zz[j] = z[min(c + j, c1 - 1)];
    if (T > 0.f) {
      if (a.uniforms) {
#pragma unroll
        for (int j = 0; j < 4; ++j) u[j] = a.uniforms[static_cast<size_t>(row) * a.ld + min(c + j, c1 - 1)];
      } else {
        uint32_t w[4] = {static_cast<uint32_t>(c >> 2), static_cast<uint32_t>(row), static_cast<uint32_t>(step),
                         static_cast<uint32_t>(step >> 32)};
        philox4x32_10(w, static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32));
#pragma unroll
        for (int j = 0; j < 4; ++j) u[j] = static_cast<float>(w[j] >> 8) * 5.9604644775390625e-08f;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (c + j >= c1) break;
      float sc = zz[j];
      if (T > 0.f) {
        const float zd = sc / T;
        const uint32_t key = fkey(zd);
        const bool kept = key > cut.x || (key == cut.x && c + j < static_cast<int>(cut.y));
        sc = kept ? gumbel_score(zd, u[j]) : -INFINITY;
      }
      best_merge(bv, bi, sc, c + j);
    }
  }
  block_best(bv, bi, sv, si);
  if (nch > 1) {
    if (threadIdx.x == 0) {
      st_dev(a.part_val + static_cast<size_t>(row) * nch + ch, bv);
      st_dev(a.part_idx + static_cast<size_t>(row) * nch + ch, bi);
      stores_done();
      last_flag = arrive_last(a.row_cnt + row, nch);
    }
    __syncthreads();
    if (!last_flag) return;
    bv = -INFINITY;
    bi = 0x7fffffff;
    for (int c = threadIdx.x; c < nch; c += blockDim.x)
      best_merge(bv, bi, ld_dev(a.part_val + static_cast<size_t>(row) * nch + c),
                 ld_dev(a.part_idx + static_cast<size_t>(row) * nch + c));
    block_best(bv, bi, sv, si);
  }
  if (threadIdx.x != 0) return;
  // a row with no candidate (every score NaN) or whose logits are marked invalid gets token -1 and
  // is not advanced, so a replay loop never embeds an id outside the vocabulary
  const bool ok = bi >= 0 && bi < a.vocab && !halted;
  const int tok = ok ? bi : -1;
  a.tokens_out[row] = tok;
  if (a.advance && ok)
    advance_row(tok, a.input_ids + row, a.positions + row, a.seq_lens + row, a.slots + row,
                a.block_table + static_cast<size_t>(row) * a.bt_stride, a.bt_stride,
                a.history ? a.history + static_cast<size_t>(row) * a.hist_ld : nullptr, a.hist_ld);
  if (a.rng && arrive_last(a.done_cnt, gridDim.x) && !halted) {
    uint64_t* r = const_cast<uint64_t*>(a.rng);
    r[1] = step + 1;
  }
}

}  // namespace gr
