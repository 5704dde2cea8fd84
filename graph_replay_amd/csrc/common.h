// Device helpers shared by the kernels: storage types, 16-byte vector loads, wave reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gr {

// Storage types. Arithmetic is fp32 everywhere; bf16/fp16 are storage and MFMA operand formats.
struct F32 {
  using S = float;
  static constexpr int kEPV = 4;  // elements per 16-byte vector
  __device__ static inline float to_f(S x) { return x; }
  __device__ static inline S from_f(float f) { return f; }
};
struct BF16 {
  using S = uint16_t;
  static constexpr int kEPV = 8;
  __device__ static inline float to_f(S x) { return __uint_as_float(static_cast<uint32_t>(x) << 16); }
  // round to nearest even (gfx950 converts in hardware: v_cvt_pk_bf16_f32)
  __device__ static inline S from_f(float f) { return __builtin_bit_cast(S, static_cast<__bf16>(f)); }
};
struct F16 {
  using S = _Float16;
  static constexpr int kEPV = 8;
  __device__ static inline float to_f(S x) { return static_cast<float>(x); }
  __device__ static inline S from_f(float f) { return static_cast<_Float16>(f); }
};

// 16-byte load/store of kEPV elements converted to/from fp32.
template <class T>
__device__ inline void load_vec(const typename T::S* p, float* out) {
  uint4 v = *reinterpret_cast<const uint4*>(p);
  if constexpr (T::kEPV == 4) {
    out[0] = __uint_as_float(v.x); out[1] = __uint_as_float(v.y);
    out[2] = __uint_as_float(v.z); out[3] = __uint_as_float(v.w);
  } else {
    const typename T::S* e = reinterpret_cast<const typename T::S*>(&v);
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = T::to_f(e[i]);
  }
}
template <class T>
__device__ inline void cvt_vec(const uint4& v, float* out) {
  if constexpr (T::kEPV == 4) {
    out[0] = __uint_as_float(v.x); out[1] = __uint_as_float(v.y);
    out[2] = __uint_as_float(v.z); out[3] = __uint_as_float(v.w);
  } else {
    const typename T::S* e = reinterpret_cast<const typename T::S*>(&v);
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = T::to_f(e[i]);
  }
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// v combined with lane l ^ 16 (xor16) or l ^ 32 (xor32) through a VALU lane swap
// (v_permlane16_swap / v_permlane32_swap: the pair's two halves land in both of its lanes), where a
// shuffle goes through LDS; both lanes of a pair get the same result, as with a shuffle
__device__ inline float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float add_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float add_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Sum over a block of blockDim.x threads (multiple of 64); every thread gets the result.
// `red` must hold blockDim.x / 64 floats of shared memory.
__device__ inline float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if (lane == 0) red[wid] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}

__device__ inline float silu(float g) { return g / (1.0f + __expf(-g)); }

// Cross-block hand-off inside one kernel, without whole-cache writeback or invalidate: the data is
// written and read with device-scope (agent) relaxed atomic stores / loads, the writer waits for
// its stores to complete (s_waitcnt) before it bumps a device-scope counter, and the reader issues
// its loads only after seeing the count. This is the memory model's agent-scope release / acquire
// for atomic data.
__device__ inline void st_dev(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<unsigned*>(p), __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_dev(int* p, int v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ inline float ld_dev(const float* p) {
  return __uint_as_float(__hip_atomic_load(reinterpret_cast<const unsigned*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ inline int ld_dev(const int* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
// two consecutive floats (8-byte aligned) in one load
__device__ inline float2 ld_dev2(const float* p) {
  const unsigned long long v =
      __hip_atomic_load(reinterpret_cast<const unsigned long long*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float(static_cast<uint32_t>(v)), __uint_as_float(static_cast<uint32_t>(v >> 32)));
}
// all of this thread's stores have completed (are visible at device scope for device-scope stores)
__device__ inline void stores_done() { __builtin_amdgcn_s_waitcnt(0); }
// counts this block in; true for exactly one block: the last of `expected` to arrive (the counter
// is reset to 0 for the next launch). Call from one thread after stores_done() + __syncthreads().
__device__ inline bool arrive_last(unsigned* counter, unsigned expected) {
  const unsigned prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const bool last = (prev == expected - 1);
  if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return last;
}

// ------------------------------------------------------------------------------------------------
// Weight prefetch into the L2 of the XCD that will read it. A batch-1 decode layer reads 30 MB of
// weights in GEMV kernels that each last only a few microseconds, so each is bound by the HBM
// latency of its first loads rather than by bandwidth, while the attention between them leaves HBM
// mostly idle. Blocks appended to a latency-bound kernel touch (one dword per 128-byte line) the
// rows that later GEMV blocks will read, on the XCD where those blocks will run: workgroups of a
// launch go round-robin over the 8 XCDs, so block b of any kernel runs on XCD b mod 8 and shares
// that XCD's 4 MB L2 with block b' of another kernel iff b = b' mod 8.
// Target t: a 1-D GEMV grid of nblk blocks; block g reads rows [g*pb, g*pb + pb) below n_rows and,
// when up_off > 0, the rows up_off + [g*pb, g*pb + pb) too (a stacked gate|up matrix); a row is
// row_bytes long. Touches are hints: no result depends on them.
constexpr int kPrefetchTargets = 3;
struct L2Prefetch {
  const char* base[kPrefetchTargets];
  int row_bytes[kPrefetchTargets];
  int pb[kPrefetchTargets];        // rows per GEMV block (per half for a gate|up matrix)
  int n_rows[kPrefetchTargets];    // rows in the GEMV's output range (gate rows for gate|up)
  int up_off[kPrefetchTargets];    // row offset of the up half, 0 if none
  int nblk[kPrefetchTargets];      // GEMV grid size
  int n;                           // targets in use (0: no prefetch blocks)
};

// Called by prefetch block `q` of `nq` (the launch's blocks [first, first + nq)); `lin` is the
// block's linear id in its launch, which fixes its XCD.
__device__ inline void l2_prefetch(const L2Prefetch& p, int lin, int first, int nq) {
  const int xcd = lin & 7;
  const int q = (lin - first) >> 3;         // index among this XCD's prefetch blocks
  const int nq_x = nq >> 3;                 // prefetch blocks per XCD (a partial last group idles)
  if (q >= nq_x) return;
  constexpr int kLine = 128, kBatch = 16;
  int items[kPrefetchTargets], lpr[kPrefetchTargets], total = 0;
  for (int t = 0; t < kPrefetchTargets; ++t) {
    if (t >= p.n) { items[t] = 0; lpr[t] = 1; continue; }
    lpr[t] = (p.row_bytes[t] + kLine - 1) / kLine;
    const int gblocks = (p.nblk[t] > xcd) ? (p.nblk[t] - 1 - xcd) / 8 + 1 : 0;   // blocks g = xcd mod 8
    items[t] = gblocks * p.pb[t] * (p.up_off[t] ? 2 : 1) * lpr[t];
    total += items[t];
  }
  const int stride = nq_x * static_cast<int>(blockDim.x);
  uint32_t acc = 0;
  for (int i0 = q * static_cast<int>(blockDim.x) + static_cast<int>(threadIdx.x); i0 < total; i0 += kBatch * stride) {
    uint32_t v[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      int i = i0 + k * stride;
      v[k] = 0;
      if (i >= total) continue;
      int t = 0;
      while (t + 1 < kPrefetchTargets && i >= items[t]) { i -= items[t]; ++t; }
      const int per_g = p.pb[t] * (p.up_off[t] ? 2 : 1) * lpr[t];
      const int g = xcd + 8 * (i / per_g);
      const int w = i % per_g;
      const int r = w / lpr[t], line = w % lpr[t];
      const int half = r / p.pb[t];
      const int row = g * p.pb[t] + (r % p.pb[t]);
      if (row >= p.n_rows[t]) continue;
      const size_t off = static_cast<size_t>(row + half * p.up_off[t]) * p.row_bytes[t] +
                         min(line * kLine, p.row_bytes[t] - 4);
      v[k] = *reinterpret_cast<const uint32_t*>(p.base[t] + off);
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) acc ^= v[k];
  }
  asm volatile("" ::"v"(acc));   // keeps the loads; nothing is stored
}

}  // namespace gr
