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
    const uint32_t lo0 = 0xD2511F53u * c[0], hi0 = __umulhi(0xD2511F53u, c[0]);
    const uint32_t lo1 = 0xCD9E8D57u * c[2], hi1 = __umulhi(0xCD9E8D57u, c[2]);
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
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
__global__ __launch_bounds__(256) void k_sample(SampleArgs a) {
  __shared__ float sv[4];
  __shared__ int si[4];
  __shared__ int last_flag;
  const int row = blockIdx.x, ch = blockIdx.y, nch = gridDim.y;
  if (a.n_rows && row >= *a.n_rows) {
    // idle row: still counted in by one block, so the step counter and its reset stay exact
    if (ch == 0 && threadIdx.x == 0 && a.rng && arrive_last(a.done_cnt, gridDim.x)) {
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
        const float uu = fminf(fmaxf(u[j], 1e-10f), 1.0f);
        sc = sc / T - logf(-logf(uu));
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
  const int tok = bi;
  a.tokens_out[row] = tok;
  if (a.advance) {
    const int len = a.seq_lens[row];
    if (len > 0) {
      const int p = a.positions[row];
      if (a.history && p < a.hist_ld) a.history[static_cast<size_t>(row) * a.hist_ld + p] = tok;
      const int np = p + 1;
      const int blk = np / 16;
      const int entry = (blk < a.bt_stride) ? a.block_table[static_cast<size_t>(row) * a.bt_stride + blk] : -1;
      if (np >= a.hist_ld || entry < 0) {
        // out of positions or of reserved blocks: the row turns into a padding row
        a.input_ids[row] = 0;
        a.positions[row] = 0;
        a.seq_lens[row] = 0;
        a.slots[row] = -1;
      } else {
        a.input_ids[row] = tok;
        a.positions[row] = np;
        a.seq_lens[row] = len + 1;
        a.slots[row] = entry * 16 + np % 16;
      }
    }
  }
  if (a.rng && arrive_last(a.done_cnt, gridDim.x)) {
    uint64_t* r = const_cast<uint64_t*>(a.rng);
    r[1] = step + 1;
  }
}

}  // namespace gr
