// Projections y = x W^T for the fused QKV, O, fused gate|up, down and LM-head matrices.
//
// The stacked matrices follow "Removing overhead: fusion, graphs and async scheduling", section
// "Fewer, larger matmuls": one matmul over [W_Q | W_K | W_V] and one over [W_gate | W_up]. Three
// kernel families cover the row counts of a step:
//   k_gemv       VALU, <= 8 token rows: every weight element is read once with 16-byte loads and
//                used for all rows; optional prologue computing x = RMSNorm(r + sum of deltas) * g
//                (the fused residual-add + RMSNorm), optional SiLU(gate) * up epilogue.
//   k_gemv_mfma  16 or 32 token rows (bf16/fp16): v_mfma_f32_16x16x32 with both operands loaded
//                straight from memory in the MFMA lane layout; the four waves split K.
//   k_gemv_stream 9-48 token rows of a wide output (the LM head): x staged in LDS once per
//                block, whole weight tiles streamed per wave.
//   k_gemm_ring  >= 33 token rows (bf16/fp16, K a multiple of 64): MFMA GEMM over an LDS ring filled
//                by direct-to-LDS loads, XCD-ordered blocks
//   k_gemm       >= 33 token rows otherwise: LDS-tiled MFMA GEMM
//   Both split K on request into fp32 partial outputs that the consumer sums in fixed order.
#pragma once
#include "common.h"
#include "sample.h"

namespace gr {

enum { EPI_F32 = 0, EPI_SILU = 1, EPI_STORE_T = 2 };

struct GemmArgs {
  int M, N, K;           // x [M][K]; W [N][K] (EPI_SILU: W [2N][K], rows N.. are `up`)
  const void* W;
  const void* bias;      // [N] in the weight dtype, or nullptr
  const void* x;         // [M][K] in the weight dtype (norm == 0)
  // norm == 1 prologue: v = r_in[m] + sum_s delta[s][m] (or embed[tok[m]] when embed != nullptr),
  // x = v / sqrt(mean(v^2) + eps) * gain, rounded to the weight dtype; block 0 stores v to r_out.
  int norm;
  const float* r_in;
  const float* delta;
  int n_delta;           // number of [M][K] partial deltas to add
  size_t delta_stride;   // floats between partials
  const void* embed;
  const int* tok;
  float* r_out;
  const void* gain;
  float eps;
  void* out;             // EPI_F32: float [ksplit][M][ldo]; EPI_SILU / EPI_STORE_T: dtype [M][ldo]
  int ldo;
  int ksplit;            // k_gemm / k_gemv_mfma: number of K ranges (gridDim.z / y)
  size_t out_split_stride;
  // k_gemv_stream with sampling (the LM head fused with the sampler): smp holds k_sample's inputs
  // (temperatures, the Philox key and step counter, token output, the in-place advance, the device
  // row count; no filters, no explicit uniforms), cand [gridDim.x][M] the blocks' best keys and
  // cand_done their arrival counter (zero between launches)
  SampleArgs smp;
  unsigned long long* cand;
  unsigned* cand_done;
};

// ------------------------------------------------------------------------------------------
// Residual-add + RMSNorm as a kernel of its own (used when the row count is too large to redo the
// norm in every projection block). One block of 256 threads per row, H <= 2048; every load of a
// phase is issued before any use and the row stays in registers. Same reduction order as the
// fused prologue of k_gemv, so both give the same bits.
template <class T>
__global__ __launch_bounds__(256) void k_add_rmsnorm(int H, const float* __restrict__ r_in,
                                                     const float* __restrict__ delta, int n_delta,
                                                     size_t delta_stride, const void* __restrict__ embed,
                                                     const int* __restrict__ tok, const int* __restrict__ row_map,
                                                     float* __restrict__ r_out, const void* __restrict__ gain,
                                                     void* __restrict__ h_out, float eps) {
  using S = typename T::S;
  constexpr int KPT = 8;
  __shared__ float red[8];
  const int m = blockIdx.x;
  const int src = row_map ? row_map[m] : m;
  const S* g = static_cast<const S*>(gain);
  float v[KPT], gk[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) gk[i] = T::to_f(g[min(static_cast<int>(threadIdx.x) + 256 * i, H - 1)]);
  if (embed) {
    const size_t eo = static_cast<size_t>(tok[src]) * H;
#pragma unroll
    for (int i = 0; i < KPT; ++i) v[i] = T::to_f(static_cast<const S*>(embed)[eo + min(static_cast<int>(threadIdx.x) + 256 * i, H - 1)]);
  } else {
    const size_t ro = static_cast<size_t>(src) * H;
#pragma unroll
    for (int i = 0; i < KPT; ++i) v[i] = r_in[ro + min(static_cast<int>(threadIdx.x) + 256 * i, H - 1)];
    // up to kDeltaBatch partials: every load issued before the first add, the adds in partial order
    constexpr int kDeltaBatch = 8;
    float db[kDeltaBatch][KPT];
#pragma unroll
    for (int s = 0; s < kDeltaBatch; ++s)
      if (s < n_delta) {
#pragma unroll
        for (int i = 0; i < KPT; ++i) db[s][i] = delta[s * delta_stride + ro + min(static_cast<int>(threadIdx.x) + 256 * i, H - 1)];
      }
#pragma unroll
    for (int s = 0; s < kDeltaBatch; ++s)
      if (s < n_delta) {
#pragma unroll
        for (int i = 0; i < KPT; ++i) v[i] += db[s][i];
      }
    for (int s = kDeltaBatch; s < n_delta; ++s) {
      float dv[KPT];
#pragma unroll
      for (int i = 0; i < KPT; ++i) dv[i] = delta[s * delta_stride + ro + min(static_cast<int>(threadIdx.x) + 256 * i, H - 1)];
#pragma unroll
      for (int i = 0; i < KPT; ++i) v[i] += dv[i];
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int k = threadIdx.x + 256 * i;
    v[i] = (k < H) ? v[i] : 0.f;
    ss += v[i] * v[i];
  }
  ss = block_sum(ss, red);
  const float inv = 1.0f / sqrtf(ss / static_cast<float>(H) + eps);
  S* h = static_cast<S*>(h_out) + static_cast<size_t>(m) * H;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int k = threadIdx.x + 256 * i;
    if (k < H) {
      if (r_out) r_out[static_cast<size_t>(m) * H + k] = v[i];
      h[k] = T::from_f(v[i] * inv * gk[i]);
    }
  }
}

// ------------------------------------------------------------------------------------------
// VALU GEMV. Block = 4 waves; wave w owns ROWS weight rows (EPI_SILU: ROWS/2 gate rows and the
// matching up rows). Lanes stride over K in 16-byte vectors, U vectors per row in flight. The
// first weight loads are issued before anything that depends on x, so the HBM stream starts at
// once; x (MT token rows) is staged in LDS as the weight dtype in chunks of KC elements. With
// norm == 1 (K <= 2048, one chunk) the prologue keeps v = r + deltas in registers, stages gain * v
// and reduces the sums of squares of all MT rows alongside; RMSNorm's 1 / rms is a per-row scalar
// of the dot product (W (g * v / rms) = (W (g * v)) / rms) and is applied in the epilogue.
template <class T, int MT, int ROWS, int U>
__global__ __launch_bounds__(256) void k_gemv(GemmArgs a, int epi) {
  using S = typename T::S;
  constexpr int EPV = T::kEPV;
  constexpr int KC = (32768 / (MT * static_cast<int>(sizeof(S)))) / (64 * EPV) * (64 * EPV);
  __shared__ __align__(16) S xs[MT * KC];
  __shared__ float red[4][MT];

  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int m0 = blockIdx.y * MT;
  const int mrows = min(MT, a.M - m0);
  const int K = a.K;
  const S* W = static_cast<const S*>(a.W);

  int rows[ROWS];
  if (epi == EPI_SILU) {
    const int j0 = (blockIdx.x * 4 + wid) * (ROWS / 2);
#pragma unroll
    for (int r = 0; r < ROWS / 2; ++r) { rows[r] = j0 + r; rows[ROWS / 2 + r] = a.N + j0 + r; }
  } else {
    const int n0 = (blockIdx.x * 4 + wid) * ROWS;
#pragma unroll
    for (int r = 0; r < ROWS; ++r) rows[r] = n0 + r;
  }
  const int nrows_total = (epi == EPI_SILU) ? 2 * a.N : a.N;

  // Loads are unconditional from clamped (always in-bounds) addresses, so the compiler can keep
  // them all in flight; vectors past the row end are skipped in the compute loop and rows past N
  // are never stored.
  uint4 wv[ROWS][U];
  auto load_w = [&](int kc0, int nv, int v0) {
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      const size_t rb = static_cast<size_t>(min(rows[r], nrows_total - 1)) * K + kc0;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int vv = min(v0 + lane + 64 * u, nv - 1);
        wv[r][u] = *reinterpret_cast<const uint4*>(W + rb + vv * EPV);
      }
    }
  };
  // the first weight vectors go out before the prologue
  load_w(0, min(KC, K) / EPV, 0);

  if (a.norm) {
    // thread t owns elements 4t .. 4t+3 of each 1024-wide slice (16-byte loads); K <= 2048
    constexpr int NS = 2;                                   // slices
    const S* g = static_cast<const S*>(a.gain);
    const int e0 = 4 * threadIdx.x;
    float gk[NS][4], v[MT][NS][4];
    size_t rowoff[MT];
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) rowoff[mm] = static_cast<size_t>(m0 + min(mm, mrows - 1)) * K;
#pragma unroll
    for (int sl = 0; sl < NS; ++sl) {
      const int k = min(e0 + 1024 * sl, K - 4);             // clamped: always in bounds
      if constexpr (sizeof(S) == 2) {
        const uint2 gv = *reinterpret_cast<const uint2*>(g + k);
        const S* ge = reinterpret_cast<const S*>(&gv);
#pragma unroll
        for (int e = 0; e < 4; ++e) gk[sl][e] = T::to_f(ge[e]);
      } else {
        const float4 gv = *reinterpret_cast<const float4*>(g + k);
        gk[sl][0] = gv.x; gk[sl][1] = gv.y; gk[sl][2] = gv.z; gk[sl][3] = gv.w;
      }
    }
    if (a.embed) {
      const S* E = static_cast<const S*>(a.embed);
#pragma unroll
      for (int mm = 0; mm < MT; ++mm) {
        const size_t eo = static_cast<size_t>(a.tok[m0 + min(mm, mrows - 1)]) * K;
#pragma unroll
        for (int sl = 0; sl < NS; ++sl) {
          const int k = min(e0 + 1024 * sl, K - 4);
          if constexpr (sizeof(S) == 2) {
            const uint2 ev = *reinterpret_cast<const uint2*>(E + eo + k);
            const S* ee = reinterpret_cast<const S*>(&ev);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[mm][sl][e] = T::to_f(ee[e]);
          } else {
            const float4 ev = *reinterpret_cast<const float4*>(E + eo + k);
            v[mm][sl][0] = ev.x; v[mm][sl][1] = ev.y; v[mm][sl][2] = ev.z; v[mm][sl][3] = ev.w;
          }
        }
      }
    } else {
#pragma unroll
      for (int mm = 0; mm < MT; ++mm)
#pragma unroll
        for (int sl = 0; sl < NS; ++sl) {
          const float4 rv = *reinterpret_cast<const float4*>(a.r_in + rowoff[mm] + min(e0 + 1024 * sl, K - 4));
          v[mm][sl][0] = rv.x; v[mm][sl][1] = rv.y; v[mm][sl][2] = rv.z; v[mm][sl][3] = rv.w;
        }
      // DB partials per round: every load of a round issued before its adds, the adds in partial
      // order (DB bounded so that the round's loads fit in registers next to the MT rows)
      constexpr int DB = MT <= 2 ? 4 : (MT <= 4 ? 2 : 1);
      for (int s0 = 0; s0 < a.n_delta; s0 += DB) {
        float4 dv[DB][MT][NS];
#pragma unroll
        for (int b = 0; b < DB; ++b)
          if (s0 + b < a.n_delta) {
            const float* dp = a.delta + (s0 + b) * a.delta_stride;
#pragma unroll
            for (int mm = 0; mm < MT; ++mm)
#pragma unroll
              for (int sl = 0; sl < NS; ++sl)
                dv[b][mm][sl] = *reinterpret_cast<const float4*>(dp + rowoff[mm] + min(e0 + 1024 * sl, K - 4));
          }
#pragma unroll
        for (int b = 0; b < DB; ++b)
          if (s0 + b < a.n_delta) {
#pragma unroll
            for (int mm = 0; mm < MT; ++mm)
#pragma unroll
              for (int sl = 0; sl < NS; ++sl) {
                v[mm][sl][0] += dv[b][mm][sl].x; v[mm][sl][1] += dv[b][mm][sl].y;
                v[mm][sl][2] += dv[b][mm][sl].z; v[mm][sl][3] += dv[b][mm][sl].w;
              }
          }
      }
    }
    float ss[MT];
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) {
      ss[mm] = 0.f;
#pragma unroll
      for (int sl = 0; sl < NS; ++sl) {
        const int k = e0 + 1024 * sl;
        const bool ok = mm < mrows && k < K;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[mm][sl][e] = ok ? v[mm][sl][e] : 0.f;
          ss[mm] += v[mm][sl][e] * v[mm][sl][e];
        }
        if (ok && blockIdx.x == 0 && a.r_out)
          *reinterpret_cast<float4*>(a.r_out + rowoff[mm] + k) =
              make_float4(v[mm][sl][0], v[mm][sl][1], v[mm][sl][2], v[mm][sl][3]);
        if (k < K) {
          // x = gain * v to LDS; the 1 / rms factor is applied to the dot products in the epilogue
#pragma unroll
          for (int e = 0; e < 4; ++e) xs[mm * KC + k + e] = T::from_f(mm < mrows ? v[mm][sl][e] * gk[sl][e] : 0.f);
        }
      }
      ss[mm] = wave_sum(ss[mm]);
    }
    if (lane == 0) {
#pragma unroll
      for (int mm = 0; mm < MT; ++mm) red[wid][mm] = ss[mm];
    }
  }

  float acc[ROWS][MT];
#pragma unroll
  for (int r = 0; r < ROWS; ++r)
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) acc[r][mm] = 0.f;

  bool preloaded = true;
  for (int kc0 = 0; kc0 < K; kc0 += KC) {
    const int kc = min(KC, K - kc0);
    const int nv = kc / EPV;  // vectors in this chunk
    if (!a.norm) {
      if (kc0) __syncthreads();
      // stage x[m0 .. m0+mrows)[kc0 .. kc0+kc) into LDS
      for (int i = threadIdx.x; i < MT * nv; i += blockDim.x) {
        const int mm = i / nv, vv = i % nv;
        uint4 val = *reinterpret_cast<const uint4*>(static_cast<const S*>(a.x) +
                                                    static_cast<size_t>(m0 + min(mm, mrows - 1)) * K + kc0 + vv * EPV);
        if (mm >= mrows) val = make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(xs + mm * KC + vv * EPV) = val;
      }
    }
    __syncthreads();
    for (int v0 = 0; v0 < nv; v0 += 64 * U) {
      if (!preloaded) load_w(kc0, nv, v0);
      preloaded = false;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int vv = v0 + lane + 64 * u;
        if (vv >= nv) continue;
        float xf[MT][EPV];
#pragma unroll
        for (int mm = 0; mm < MT; ++mm) load_vec<T>(xs + mm * KC + vv * EPV, xf[mm]);
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
          float wf[EPV];
          cvt_vec<T>(wv[r][u], wf);
#pragma unroll
          for (int mm = 0; mm < MT; ++mm)
#pragma unroll
            for (int e = 0; e < EPV; ++e) acc[r][mm] = fmaf(wf[e], xf[mm][e], acc[r][mm]);
        }
      }
    }
  }

#pragma unroll
  for (int r = 0; r < ROWS; ++r)
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) acc[r][mm] = wave_sum(acc[r][mm]);
  if (a.norm) {
    // red[][] was written before the staging barrier
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) {
      const float inv = 1.0f / sqrtf((red[0][mm] + red[1][mm] + red[2][mm] + red[3][mm]) / static_cast<float>(K) + a.eps);
#pragma unroll
      for (int r = 0; r < ROWS; ++r) acc[r][mm] *= inv;
    }
  }

  if (lane == 0) {
    if (epi == EPI_SILU) {
      S* out = static_cast<S*>(a.out);
#pragma unroll
      for (int r = 0; r < ROWS / 2; ++r) {
        if (rows[r] >= a.N) continue;
        for (int mm = 0; mm < mrows; ++mm)
          out[static_cast<size_t>(m0 + mm) * a.ldo + rows[r]] = T::from_f(silu(acc[r][mm]) * acc[ROWS / 2 + r][mm]);
      }
    } else {
      float* out = static_cast<float*>(a.out);
      const S* b = static_cast<const S*>(a.bias);
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        if (rows[r] >= a.N) continue;
        const float bb = b ? T::to_f(b[rows[r]]) : 0.f;
        for (int mm = 0; mm < mrows; ++mm) out[static_cast<size_t>(m0 + mm) * a.ldo + rows[r]] = acc[r][mm] + bb;
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// MFMA fragment types (gfx950 v_mfma_f32_16x16x32_{bf16,f16}). Lane l of a 16x32 A fragment holds
// row l % 16, k = 8 * (l / 16) .. + 8; the B fragment holds column l % 16 with the same k slots;
// the 16x16 fp32 result holds rows 4 * (l / 16) + i (i = 0..3) of column l % 16.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <class T>
__device__ inline f32x4_t mfma16x16x32(const uint4& a, const uint4& b, f32x4_t c) {
  if constexpr (sizeof(typename T::S) == 2 && T::kEPV == 8 && __is_same(T, BF16)) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
}

// 16x16x16 variant: lane l holds k = 4 * (l / 16) .. + 4 of its row (A) or column (B)
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

// two fp32 values rounded to the 16-bit storage type, packed low then high
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
template <class T>
__device__ inline uint32_t pack2(float x, float y) {
  if constexpr (__is_same(T, BF16)) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{x, y}, bf16x2_t));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{x, y}, f16x2_t));
  }
}

// s_waitcnt with only a vector-memory count (expcnt and lgkmcnt left at "no wait"), gfx9 encoding
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

typedef __attribute__((address_space(3))) void lds_void_t;

// One 16-byte direct-to-LDS load per lane (global_load_lds_dwordx4): lane l writes the 16 bytes at
// `g` to LDS address lds + 16 l. It is issued as inline assembly so that the compiler, which cannot
// tell ring slots apart, does not put a wait for every outstanding LDS load in front of each LDS
// read; the caller waits with wait_vmcnt and a barrier before reading the slot. (The compiler does
// not count these loads, and no other vector-memory load is in flight around them.)
__device__ inline void lds_load16(const void* g, void* lds) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)lds)));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(base), "v"(g) : "memory");
}

// MFMA GEMM for many token rows: out[m][n] = sum_k x[m][k] W[n][k], both operands K-contiguous.
// Block tile BN weight rows x BM tokens, NWN x NWM waves each owning a WN x WM sub-tile of 16x16
// MFMA tiles (v_mfma_f32_16x16x32). K goes in steps of BK = 64 (a tile row is 128 bytes = 8 vectors)
// through a ring of NS LDS stages filled by direct-to-LDS loads, so NS - 1 steps are in flight
// without staging registers; with NS = 2 two blocks fit per CU. The 16-byte vector c of tile row r
// sits in slot c ^ ((r >> 1) & 7) of the row (each load instruction covers 8 rows and takes its
// lanes' sources in that order): the 16 lanes that read one MFMA fragment column then hit 16
// distinct bank groups. One wait + barrier per k-step: after it, step s is in LDS for every wave
// and nobody reads step s - 1, whose slot takes step s + NS - 1.
// Block order is XCD-aware: block b runs on XCD b % 8 (round-robin dispatch), and the blocks of one
// XCD take all m tiles of an n tile before the next, so a weight tile is read into one L2.
// EPI_SILU: within each wave the first WN/2 rows are gate rows and the last WN/2 the matching up
// rows, so SiLU(gate) * up is formed in registers. gridDim.z splits K (EPI_F32 partial outputs).
template <class T, int BN, int BM, int NWN, int NWM, int NS>
__global__ __launch_bounds__(64 * NWN * NWM) void k_gemm_ring(GemmArgs a, int epi, int n_tiles, int m_tiles) {
  using S = typename T::S;
  constexpr int BK = 64, NW = NWN * NWM;
  constexpr int WN = BN / NWN, WM = BM / NWM;
  constexpr int TN = WN / 16, TM = WM / 16;
  constexpr int WI = BN / 8 / NW, XI = BM / 8 / NW;   // load instructions per wave per k-step
  constexpr int LPS = WI + XI;
  constexpr int STAGE = (BN + BM) * 128;                // bytes per stage
  static_assert(WN % 32 == 0 && WM % 16 == 0, "tile shape");
  static_assert(WI * NW * 8 == BN && XI * NW * 8 == BM, "rows must split evenly over the waves");
  static_assert(LPS * (NS - 2) < 64 && NS >= 2, "vmcnt range");
  __shared__ __align__(16) unsigned char ring[NS * STAGE];

  const int b = blockIdx.x;
  const int slot = b >> 3;
  const int tn = (b & 7) + 8 * (slot / m_tiles), tm = slot % m_tiles;
  if (tn >= n_tiles) return;
  const int lane = threadIdx.x & 63, wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wid % NWN, wm = wid / NWN;
  const int K = a.K;
  const bool silu_epi = (epi == EPI_SILU);
  const int m0 = tm * BM;
  const S* W = static_cast<const S*>(a.W);
  const S* X = static_cast<const S*>(a.x);

  auto wrow_of = [&](int R) -> int {                    // tile row -> weight row (clamped)
    if (silu_epi) {
      const int w = R / WN, r = R % WN;
      const int j = min(tn * (BN / 2) + w * (WN / 2) + (r % (WN / 2)), a.N - 1);
      return (r < WN / 2) ? j : a.N + j;
    }
    return min(tn * BN + R, a.N - 1);
  };
  const int ksteps = K / BK;
  const int per = (ksteps + gridDim.z - 1) / gridDim.z;
  const int ks0 = blockIdx.z * per, ks1 = min(ksteps, ks0 + per);
  const int n = max(0, ks1 - ks0);

  // this lane's source for each of its load instructions (row r = 8 q + lane / 8, slot lane % 8);
  // rows past N or M read a clamped valid row, and their outputs are never stored
  const S* wsrc[WI];
  const S* xsrc[XI];
#pragma unroll
  for (int i = 0; i < WI; ++i) {
    const int q = wid + NW * i, r = 8 * q + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    wsrc[i] = W + static_cast<size_t>(wrow_of(r)) * K + c * 8;
  }
#pragma unroll
  for (int i = 0; i < XI; ++i) {
    const int q = wid + NW * i, r = 8 * q + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    xsrc[i] = X + static_cast<size_t>(min(m0 + r, a.M - 1)) * K + c * 8;
  }
  auto issue = [&](int s) {                             // k-step ks0 + s into ring slot s % NS
    unsigned char* st = ring + (s % NS) * STAGE;
    const int k0 = (ks0 + s) * BK;
#pragma unroll
    for (int i = 0; i < WI; ++i) lds_load16(wsrc[i] + k0, st + (wid + NW * i) * 1024);
#pragma unroll
    for (int i = 0; i < XI; ++i) lds_load16(xsrc[i] + k0, st + BN * 128 + (wid + NW * i) * 1024);
  };

  f32x4_t acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < n) issue(s);
  const int frow = lane & 15, kq = lane >> 4;
  for (int s = 0; s < n; ++s) {
    // this wave's loads of step s are done once at most NS - 2 later steps are outstanding
    if (s + NS - 2 < n) wait_vmcnt<LPS * (NS - 2)>();
    else wait_vmcnt<0>();
    __syncthreads();
    if (s + NS - 1 < n) issue(s + NS - 1);
    const unsigned char* st = ring + (s % NS) * STAGE;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int c = kk * 4 + kq;                        // k vector of this lane's fragment slots
      uint4 af[TN], bf[TM];
#pragma unroll
      for (int i = 0; i < TN; ++i) {
        const int r = wn * WN + i * 16 + frow;
        af[i] = *reinterpret_cast<const uint4*>(st + r * 128 + ((c ^ ((r >> 1) & 7)) << 4));
      }
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const int r = wm * WM + j * 16 + frow;
        bf[j] = *reinterpret_cast<const uint4*>(st + BN * 128 + r * 128 + ((c ^ ((r >> 1) & 7)) << 4));
      }
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[i][j] = mfma16x16x32<T>(af[i], bf[j], acc[i][j]);
    }
  }
  // (the last step waited for vmcnt 0: no load is in flight past this point)

  const int col = lane & 15, rbase = 4 * (lane >> 4);
  if (silu_epi) {
    S* out = static_cast<S*>(a.out);
#pragma unroll
    for (int i = 0; i < TN / 2; ++i) {
      const int j0 = tn * (BN / 2) + wn * (WN / 2) + i * 16 + rbase;
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const int m = m0 + wm * WM + j * 16 + col;
        if (m >= a.M) continue;
        S v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = T::from_f(silu(acc[i][j][e]) * acc[i + TN / 2][j][e]);
        S* dst = out + static_cast<size_t>(m) * a.ldo + j0;
        if (j0 + 3 < a.N) {
          *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(v);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (j0 + e < a.N) dst[e] = v[e];
        }
      }
    }
  } else {
    const S* bias = (blockIdx.z == 0) ? static_cast<const S*>(a.bias) : nullptr;
#pragma unroll
    for (int i = 0; i < TN; ++i) {
      const int n0 = tn * BN + wn * WN + i * 16 + rbase;
      float bb[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) bb[e] = (bias && n0 + e < a.N) ? T::to_f(bias[n0 + e]) : 0.f;
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const int m = m0 + wm * WM + j * 16 + col;
        if (m >= a.M) continue;
        if (epi == EPI_STORE_T) {
          S v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = T::from_f(acc[i][j][e] + bb[e]);
          S* dst = static_cast<S*>(a.out) + static_cast<size_t>(m) * a.ldo + n0;
          if (n0 + 3 < a.N) {
            *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(v);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (n0 + e < a.N) dst[e] = v[e];
          }
        } else {
          float* dst = static_cast<float*>(a.out) + blockIdx.z * a.out_split_stride + static_cast<size_t>(m) * a.ldo + n0;
          const float4 v = make_float4(acc[i][j][0] + bb[0], acc[i][j][1] + bb[1], acc[i][j][2] + bb[2],
                                       acc[i][j][3] + bb[3]);
          if (n0 + 3 < a.N) {
            *reinterpret_cast<float4*>(dst) = v;
          } else {
            const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (n0 + e < a.N) dst[e] = vv[e];
          }
        }
      }
    }
  }
}

// Skinny MFMA GEMV: block = 4 waves over RT tiles of 16 weight rows (EPI_SILU: each tile is 8 gate
// rows and the matching 8 up rows) and MB 16-token tiles; wave w accumulates k-steps w, w+4, ... and
// the partial tiles are summed in wave order through LDS. One activation fragment feeds RT MFMAs,
// so the activation loads (from L2) are amortised over RT weight tiles. gridDim.y splits K into
// a.ksplit ranges (EPI_F32 only) whose fp32 partials go to out + split * out_split_stride. UN k-steps
// per wave are loaded at once.
template <class T, int MB, int UN, int RT>
__global__ __launch_bounds__(256) void k_gemv_mfma(GemmArgs a, int epi) {
  using S = typename T::S;
  __shared__ f32x4_t part[4][RT][MB][64];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int K = a.K;
  const S* W = static_cast<const S*>(a.W);
  const S* X = static_cast<const S*>(a.x);
  const int nrows_total = (epi == EPI_SILU) ? 2 * a.N : a.N;
  const uint4 zero4 = make_uint4(0, 0, 0, 0);
  // weight row of this lane in each tile (clamped, so every load is in bounds; out-of-range rows are
  // zeroed by select and never stored)
  const S* wp[RT];
  bool wok[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    int wrow;
    if (epi == EPI_SILU) {
      const int j = (blockIdx.x * RT + r) * 8 + (lane & 7);
      wrow = ((lane & 15) < 8) ? j : a.N + j;
      wok[r] = j < a.N;
    } else {
      wrow = (blockIdx.x * RT + r) * 16 + (lane & 15);
      wok[r] = wrow < a.N;
    }
    wp[r] = W + static_cast<size_t>(min(wrow, nrows_total - 1)) * K + 8 * (lane >> 4);
  }
  const int ksteps = K / 32;
  const int per = (ksteps + a.ksplit - 1) / a.ksplit;
  const int ks0 = blockIdx.y * per, ks1 = min(ksteps, ks0 + per);
  const int koff = 8 * (lane >> 4);

  f32x4_t acc[RT][MB];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int t = 0; t < MB; ++t) acc[r][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const S* xp[MB];
  bool xok[MB];
#pragma unroll
  for (int t = 0; t < MB; ++t) {
    const int m = t * 16 + (lane & 15);
    xok[t] = m < a.M;
    xp[t] = X + static_cast<size_t>(xok[t] ? m : a.M - 1) * K + koff;
  }
  int ks = ks0 + wid;
  for (; ks + 4 * (UN - 1) < ks1; ks += 4 * UN) {
    uint4 av[UN][RT], bv[UN][MB];
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int k = (ks + 4 * u) * 32;
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        av[u][r] = *reinterpret_cast<const uint4*>(wp[r] + k);
        if (!wok[r]) av[u][r] = zero4;
      }
#pragma unroll
      for (int t = 0; t < MB; ++t) {
        bv[u][t] = *reinterpret_cast<const uint4*>(xp[t] + k);
        if (!xok[t]) bv[u][t] = zero4;
      }
    }
#pragma unroll
    for (int u = 0; u < UN; ++u)
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int t = 0; t < MB; ++t) acc[r][t] = mfma16x16x32<T>(av[u][r], bv[u][t], acc[r][t]);
  }
  for (; ks < ks1; ks += 4) {
    const int k = ks * 32;
    uint4 av[RT], bv[MB];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      av[r] = *reinterpret_cast<const uint4*>(wp[r] + k);
      if (!wok[r]) av[r] = zero4;
    }
#pragma unroll
    for (int t = 0; t < MB; ++t) {
      bv[t] = *reinterpret_cast<const uint4*>(xp[t] + k);
      if (!xok[t]) bv[t] = zero4;
    }
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int t = 0; t < MB; ++t) acc[r][t] = mfma16x16x32<T>(av[r], bv[t], acc[r][t]);
  }
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int t = 0; t < MB; ++t) part[wid][r][t][lane] = acc[r][t];
  __syncthreads();
  // wave r' of the block finishes tile r' (RT <= 4), summing the four waves in order
  const int r = wid;
  if (r >= RT) return;
#pragma unroll
  for (int t = 0; t < MB; ++t) {
    f32x4_t sum = part[0][r][t][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) sum += part[w][r][t][lane];
    acc[0][t] = sum;
  }
  const int col = lane & 15;          // token within the tile
  const int rbase = 4 * (lane >> 4);  // first of the 4 weight rows this lane holds
  if (epi == EPI_SILU) {
    // lanes 0..31 hold gate rows 0..7, lanes 32..63 the matching up rows 8..15
    S* out = static_cast<S*>(a.out);
#pragma unroll
    for (int t = 0; t < MB; ++t) {
      f32x4_t up;
#pragma unroll
      for (int i = 0; i < 4; ++i) up[i] = __shfl(acc[0][t][i], lane + 32, 64);
      const int m = t * 16 + col;
      if (lane < 32 && m < a.M) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = (blockIdx.x * RT + r) * 8 + rbase + i;
          if (j < a.N) out[static_cast<size_t>(m) * a.ldo + j] = T::from_f(silu(acc[0][t][i]) * up[i]);
        }
      }
    }
  } else {
    float* out = static_cast<float*>(a.out) + blockIdx.y * a.out_split_stride;
    const S* b = (blockIdx.y == 0) ? static_cast<const S*>(a.bias) : nullptr;
#pragma unroll
    for (int t = 0; t < MB; ++t) {
      const int m = t * 16 + col;
      if (m >= a.M) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = (blockIdx.x * RT + r) * 16 + rbase + i;
        if (n < a.N) out[static_cast<size_t>(m) * a.ldo + n] = acc[0][t][i] + (b ? T::to_f(b[n]) : 0.f);
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// Streaming skinny MFMA GEMV for a wide output over 9-48 token rows (the LM head): the MB * 16
// token rows of x go to LDS once per block, then every wave owns whole 16-row weight tiles (tiles
// w, w + W, ... for wave w of W in the grid) and streams each tile's K in chunks of kStreamCh
// k-steps, the next chunk's weight loads in flight while the current chunk's MFMAs run (NWV waves
// per block, CH k-steps per chunk). In LDS,
// the 16-byte chunk c of row m sits at chunk c ^ (m & 15), so the 16 rows a lane group reads at
// one k offset fall in distinct banks. fp32 out [M][ldo]; no bias, no K split; K a multiple of
// 32 * CH and at most KMAX (LDS: MB * 16 * KMAX elements; two blocks per CU up to 64 KiB).
//
// SAMPLE: the sampler fused into the epilogue ("Removing overhead: fusion, graphs and async
// scheduling", section "Fewer, larger matmuls", lists the LM head fused with sampling among the
// fusions production engines make). A lane's tile output is four consecutive vocabulary rows of one
// token row, the four columns of one Philox call, so each lane scores its logits exactly as
// k_sample would (z at temperature 0, else z / T plus the Gumbel noise of the (row, column)
// uniform), keeps the best score_key per token row, and the block stores one key per row. The last
// block to arrive takes each row's best key, writes the token, runs advance_row and moves the step
// counter on, as k_sample's last blocks do, so the tokens are bit-identical to k_sample's on the
// stored logits. The logits are still stored.
template <class T, int MB, int NWV, int CH, int KMAX, bool SAMPLE>
__global__ __launch_bounds__(64 * NWV, MB * 16 * KMAX * 2 <= 65536 ? 2 : 1) void k_gemv_stream(GemmArgs a) {
  using S = typename T::S;
  static_assert(sizeof(S) == 2, "16-bit types");
  __shared__ __align__(16) S xs[MB * 16 * KMAX];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int K = a.K;
  const int cpt = K / (32 * CH);                     // chunks per tile
  const int ntiles = (a.N + 15) / 16;
  const int nwaves = gridDim.x * NWV;
  const int tile0 = blockIdx.x * NWV + wid;
  const int nseq = tile0 < ntiles ? ((ntiles - 1 - tile0) / nwaves + 1) * cpt : 0;
  const S* W = static_cast<const S*>(a.W);
  uint4 wa[CH], wb[CH];
  // the weight chunk q of this wave's sequence (rows past N clamped: loaded, never stored)
  auto load = [&](uint4(&w)[CH], int q) {
    const int row = min((tile0 + (q / cpt) * nwaves) * 16 + col, a.N - 1);
    const S* p = W + static_cast<size_t>(row) * K + (q % cpt) * (32 * CH) + 8 * grp;
#pragma unroll
    for (int j = 0; j < CH; ++j) w[j] = *reinterpret_cast<const uint4*>(p + 32 * j);
  };
  if (nseq > 0) load(wa, 0);
  // x -> LDS (zero rows past M), behind the first chunk's loads
  const int nch = K / 8;
  const S* X = static_cast<const S*>(a.x);
  for (int i = threadIdx.x; i < MB * 16 * nch; i += 64 * NWV) {
    const int m = i / nch, c = i % nch;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (m < a.M) v = *reinterpret_cast<const uint4*>(X + static_cast<size_t>(m) * K + 8 * c);
    *reinterpret_cast<uint4*>(xs + m * K + 8 * (c ^ (m & 15))) = v;
  }
  __syncthreads();
  f32x4_t acc[MB];
#pragma unroll
  for (int t = 0; t < MB; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // fused sampler state of this lane's token rows t * 16 + col
  const int n_samp = SAMPLE ? (a.smp.n_rows ? min(*a.smp.n_rows, a.M) : a.M) : 0;
  const uint64_t seed = SAMPLE ? (a.smp.rng ? a.smp.rng[0] : a.smp.seed) : 0ull;
  const uint64_t stepc = SAMPLE ? (a.smp.rng ? a.smp.rng[1] : a.smp.step) : 0ull;
  float temp[MB];
  unsigned long long best[MB];
#pragma unroll
  for (int t = 0; t < MB; ++t) {
    const int m = t * 16 + col;
    temp[t] = (SAMPLE && m < n_samp && a.smp.temperature) ? a.smp.temperature[m] : 0.f;
    best[t] = 0ull;
  }
  auto compute = [&](const uint4(&w)[CH], int q) {
    const int ks0 = (q % cpt) * CH;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int c = (ks0 + j) * 4 + grp;
#pragma unroll
      for (int t = 0; t < MB; ++t) {
        const uint4 xv = *reinterpret_cast<const uint4*>(xs + (t * 16 + col) * K + 8 * (c ^ col));
        acc[t] = mfma16x16x32<T>(w[j], xv, acc[t]);
      }
    }
    if (q % cpt == cpt - 1) {   // the tile's last chunk: lane holds rows 4 grp + i of token col
      const int nb = (tile0 + (q / cpt) * nwaves) * 16 + 4 * grp;
      float* out = static_cast<float*>(a.out);
#pragma unroll
      for (int t = 0; t < MB; ++t) {
        const int m = t * 16 + col;
        if (m < a.M) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (nb + i < a.N) out[static_cast<size_t>(m) * a.ldo + nb + i] = acc[t][i];
        }
        if (SAMPLE && m < n_samp) {
          float u[4] = {1.f, 1.f, 1.f, 1.f};
          if (temp[t] > 0.f) {
            uint32_t w4[4] = {static_cast<uint32_t>(nb >> 2), static_cast<uint32_t>(m), static_cast<uint32_t>(stepc),
                              static_cast<uint32_t>(stepc >> 32)};
            philox4x32_10(w4, static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32));
#pragma unroll
            for (int i = 0; i < 4; ++i) u[i] = static_cast<float>(w4[i] >> 8) * 5.9604644775390625e-08f;
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (nb + i < a.N) {
              const float sc = temp[t] > 0.f ? gumbel_score(acc[t][i] / temp[t], u[i]) : acc[t][i];
              const unsigned long long k = score_key(sc, nb + i);
              best[t] = k > best[t] ? k : best[t];
            }
          }
        }
        acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  for (int q = 0; q < nseq; q += 2) {
    if (q + 1 < nseq) load(wb, q + 1);
    compute(wa, q);
    if (q + 1 < nseq) {
      if (q + 2 < nseq) load(wa, q + 2);
      compute(wb, q + 1);
    }
  }
  if constexpr (SAMPLE) {
    // the block's best key per token row: the four lane groups of a wave, then the waves
    constexpr int R = MB * 16;
    // the reduction's LDS reuses the activation rows (every wave is past its last product after the
    // barrier), so the block keeps the LDS footprint of the plain kernel
    static_assert(sizeof(unsigned long long) * (NWV * R + 1) <= sizeof(S) * MB * 16 * KMAX, "LDS reuse");
    __syncthreads();
    unsigned long long (*sbest)[R] = reinterpret_cast<unsigned long long (*)[R]>(xs);
    int& s_last = *reinterpret_cast<int*>(reinterpret_cast<unsigned long long*>(xs) + NWV * R);
#pragma unroll
    for (int t = 0; t < MB; ++t) {
      unsigned long long b = best[t];
#pragma unroll
      for (int o = 16; o < 64; o <<= 1) {
        const uint32_t lo = __shfl_xor(static_cast<uint32_t>(b), o, 64);
        const uint32_t hi = __shfl_xor(static_cast<uint32_t>(b >> 32), o, 64);
        const unsigned long long w = (static_cast<unsigned long long>(hi) << 32) | lo;
        b = w > b ? w : b;
      }
      if (grp == 0) sbest[wid][t * 16 + col] = b;
    }
    __syncthreads();
    if (threadIdx.x < R) {
      unsigned long long b = 0ull;
#pragma unroll
      for (int w = 0; w < NWV; ++w) b = sbest[w][threadIdx.x] > b ? sbest[w][threadIdx.x] : b;
      __hip_atomic_store(a.cand + static_cast<size_t>(blockIdx.x) * R + threadIdx.x, b, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
    stores_done();
    __syncthreads();
    if (threadIdx.x == 0) s_last = arrive_last(a.cand_done, gridDim.x);
    __syncthreads();
    if (!s_last) return;
    // the last block: row m's best key over all blocks (wave w takes rows w, w + NWV, ...), every
    // load of the wave issued before the first comparison (fixed trip counts; the grid has at most
    // 512 blocks)
    constexpr int RPW = (R + NWV - 1) / NWV;
    unsigned long long kk[RPW][8];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int m = wid + NWV * r;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int blk = lane + 64 * j;
        kk[r][j] = (m < n_samp && blk < static_cast<int>(gridDim.x))
                       ? __hip_atomic_load(a.cand + static_cast<size_t>(blk) * R + m, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT)
                       : 0ull;
      }
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int m = wid + NWV * r;
      unsigned long long b = 0ull;
#pragma unroll
      for (int j = 0; j < 8; ++j) b = kk[r][j] > b ? kk[r][j] : b;
      b = wave_max_u64(b);
      if (m < n_samp && lane == 0) {
        const int idx = b ? static_cast<int>(~static_cast<uint32_t>(b)) : -1;
        // no candidate (every score NaN): token -1 and no advance, as in k_sample
        const bool ok = idx >= 0 && idx < a.N;
        a.smp.tokens_out[m] = ok ? idx : -1;
        if (a.smp.advance && ok)
          advance_row(idx, a.smp.input_ids + m, a.smp.positions + m, a.smp.seq_lens + m, a.smp.slots + m,
                      a.smp.block_table + static_cast<size_t>(m) * a.smp.bt_stride, a.smp.bt_stride,
                      a.smp.history ? a.smp.history + static_cast<size_t>(m) * a.smp.hist_ld : nullptr,
                      a.smp.hist_ld);
      }
    }
    if (threadIdx.x == 0 && a.smp.rng) {
      uint64_t* r = const_cast<uint64_t*>(a.smp.rng);
      r[1] = stepc + 1;
    }
  }
}

// ------------------------------------------------------------------------------------------
// LDS-tiled MFMA GEMM for many token rows. Tile BN weight rows x BM tokens, BK = 32, 4 waves as
// 2 (weight rows) x 2 (tokens). EPI_SILU maps the first BN/2 tile rows to gate rows and the last
// BN/2 to the matching up rows. Block index: x = weight-row tile, y = token tile, z = K split.
template <class T, int BN, int BM>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs a, int epi) {
  using S = typename T::S;
  constexpr int BK = 32, LDK = BK + 8;            // padded LDS rows (elements)
  constexpr int WN = BN / 2, WM = BM / 2;         // wave tile
  constexpr int TN = WN / 16, TM = WM / 16;       // MFMA tiles per wave
  constexpr size_t kTileBytes = 2 * (BN + BM) * LDK * sizeof(S);
  constexpr size_t kExBytes = sizeof(float) * WN * BM;
  __shared__ __align__(16) unsigned char smem[kTileBytes > kExBytes ? kTileBytes : kExBytes];
  S (*ws)[BN * LDK] = reinterpret_cast<S (*)[BN * LDK]>(smem);
  S (*xs_)[BM * LDK] = reinterpret_cast<S (*)[BM * LDK]>(smem + 2 * BN * LDK * sizeof(S));
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wn = wid & 1, wm = wid >> 1;
  const int K = a.K;
  const S* W = static_cast<const S*>(a.W);
  const S* X = static_cast<const S*>(a.x);
  const int nrows_total = (epi == EPI_SILU) ? 2 * a.N : a.N;
  const int m0 = blockIdx.y * BM;

  auto wrow_of = [&](int r) -> int {  // tile row -> weight row
    if (epi == EPI_SILU) {
      const int half = BN / 2;
      const int j = blockIdx.x * half + (r % half);
      return (r < half) ? j : a.N + j;
    }
    return blockIdx.x * BN + r;
  };
  const int ksteps = K / BK;
  const int per = (ksteps + a.ksplit - 1) / a.ksplit;
  const int ks0 = blockIdx.z * per, ks1 = min(ksteps, ks0 + per);

  // global -> register staging: each thread moves (BN + BM) * BK / 8 / 256 vectors per k-step
  constexpr int WV = BN * BK / 8 / 256, XV = BM * BK / 8 / 256;
  static_assert(WV >= 1 && XV >= 1, "tile too small for 256 threads");
  uint4 wreg[WV], xreg[XV];
  auto load_tiles = [&](int ks) {
    const int k0 = ks * BK;
#pragma unroll
    for (int i = 0; i < WV; ++i) {
      const int idx = threadIdx.x + 256 * i, r = idx >> 2, c = (idx & 3) * 8;
      const int wr = wrow_of(r);
      wreg[i] = *reinterpret_cast<const uint4*>(W + static_cast<size_t>(min(wr, nrows_total - 1)) * K + k0 + c);
      if (wr >= nrows_total) wreg[i] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < XV; ++i) {
      const int idx = threadIdx.x + 256 * i, r = idx >> 2, c = (idx & 3) * 8;
      const int m = m0 + r;
      xreg[i] = *reinterpret_cast<const uint4*>(X + static_cast<size_t>(min(m, a.M - 1)) * K + k0 + c);
      if (m >= a.M) xreg[i] = make_uint4(0, 0, 0, 0);
    }
  };
  auto store_tiles = [&](int buf) {
#pragma unroll
    for (int i = 0; i < WV; ++i) {
      const int idx = threadIdx.x + 256 * i, r = idx >> 2, c = (idx & 3) * 8;
      *reinterpret_cast<uint4*>(&ws[buf][r * LDK + c]) = wreg[i];
    }
#pragma unroll
    for (int i = 0; i < XV; ++i) {
      const int idx = threadIdx.x + 256 * i, r = idx >> 2, c = (idx & 3) * 8;
      *reinterpret_cast<uint4*>(&xs_[buf][r * LDK + c]) = xreg[i];
    }
  };

  f32x4_t acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (ks0 < ks1) {
    load_tiles(ks0);
    store_tiles(0);
  }
  __syncthreads();
  int buf = 0;
  for (int ks = ks0; ks < ks1; ++ks) {
    const bool more = ks + 1 < ks1;
    if (more) load_tiles(ks + 1);
    uint4 af[TN], bfr[TM];
    const int koff = 8 * (lane >> 4);
#pragma unroll
    for (int i = 0; i < TN; ++i)
      af[i] = *reinterpret_cast<const uint4*>(&ws[buf][(wn * WN + i * 16 + (lane & 15)) * LDK + koff]);
#pragma unroll
    for (int j = 0; j < TM; ++j)
      bfr[j] = *reinterpret_cast<const uint4*>(&xs_[buf][(wm * WM + j * 16 + (lane & 15)) * LDK + koff]);
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) acc[i][j] = mfma16x16x32<T>(af[i], bfr[j], acc[i][j]);
    if (more) {
      store_tiles(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
  }

  const int col = lane & 15, rbase = 4 * (lane >> 4);
  if (epi == EPI_SILU) {
    // wave wn = 1 holds the up rows matching wave wn = 0's gate rows: exchange through LDS
    __syncthreads();
    float* ex = reinterpret_cast<float*>(smem);   // WN * BM floats
    if (wn == 1) {
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) ex[(i * 16 + rbase + e) * BM + wm * WM + j * 16 + col] = acc[i][j][e];
    }
    __syncthreads();
    if (wn == 0) {
      S* out = static_cast<S*>(a.out);
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) {
          const int m = m0 + wm * WM + j * 16 + col;
          if (m >= a.M) continue;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int jj = blockIdx.x * (BN / 2) + i * 16 + rbase + e;
            const float up = ex[(i * 16 + rbase + e) * BM + wm * WM + j * 16 + col];
            if (jj < a.N) out[static_cast<size_t>(m) * a.ldo + jj] = T::from_f(silu(acc[i][j][e]) * up);
          }
        }
    }
  } else {
    float* outf = static_cast<float*>(a.out) + blockIdx.z * a.out_split_stride;
    S* outt = static_cast<S*>(a.out);
    const S* b = (blockIdx.z == 0) ? static_cast<const S*>(a.bias) : nullptr;
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const int m = m0 + wm * WM + j * 16 + col;
        if (m >= a.M) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int n = blockIdx.x * BN + wn * WN + i * 16 + rbase + e;
          if (n >= a.N) continue;
          const float v = acc[i][j][e] + (b ? T::to_f(b[n]) : 0.f);
          if (epi == EPI_STORE_T) outt[static_cast<size_t>(m) * a.ldo + n] = T::from_f(v);
          else outf[static_cast<size_t>(m) * a.ldo + n] = v;
        }
      }
  }
}

}  // namespace gr
