// C ABI of the mixture-of-experts layer (include/moe.h): argument checks, the workspace layout,
// and the four launches of moe.h's kernels on the caller's stream.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "moe.h"
#include "../../include/moe.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) noexcept {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  try {
    g_err = buf;
  } catch (...) {
    // no memory for the message: the code still reports the failure
  }
  return code;
}

constexpr size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct MoeLayout {
  size_t sorted, bexp, brank, npad, act, rows, total;
  int m_max;
};

// -1 when out of range
long long rows_for(long long total, long long E, long long bm) {
  if (total < 0 || E < 1 || E > MOE_MAX_EXPERTS || bm < 1 || bm > 65536) return -1;
  const long long m = total + E * (bm - 1);
  const long long r = (m + bm - 1) / bm * bm;
  return r > 0x7fffffffLL ? -1 : r;
}

// checks a layer's sizes; fills the workspace layout
int check_layer(const moe_layer* L, MoeLayout* lay) {
  if (!L) return fail(STEP_EINVAL, "layer is NULL");
  if (L->dtype != STEP_BF16 && L->dtype != STEP_F16)
    return fail(STEP_EUNSUPPORTED, "moe dtype %d: only STEP_BF16 and STEP_F16 have kernels", L->dtype);
  if (L->n_tokens < 0 || L->top_k < 1 || L->num_experts < 1 || L->num_experts > MOE_MAX_EXPERTS)
    return fail(STEP_EINVAL, "moe sizes: n_tokens %d, top_k %d, num_experts %d (1..%d)", L->n_tokens, L->top_k,
                L->num_experts, MOE_MAX_EXPERTS);
  if (L->hidden <= 0 || L->hidden % 32 || L->inter <= 0 || L->inter % 32)
    return fail(STEP_EINVAL, "moe hidden %d and inter %d must be positive multiples of 32", L->hidden, L->inter);
  const long long total = static_cast<long long>(L->n_tokens) * L->top_k;
  if (total > 0x7fffffffLL) return fail(STEP_EINVAL, "n_tokens * top_k does not fit an int32");
  const long long m = rows_for(total, L->num_experts, MOE_BLOCK_M);
  if (m < 0) return fail(STEP_EINVAL, "grouped rows do not fit an int32");
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += align256(bytes); return o; };
  lay->m_max = static_cast<int>(m);
  lay->sorted = take(sizeof(int32_t) * static_cast<size_t>(m));
  lay->bexp = take(sizeof(int32_t) * static_cast<size_t>(m / MOE_BLOCK_M));
  lay->brank = take(sizeof(int32_t) * static_cast<size_t>(m / MOE_BLOCK_M));
  lay->npad = take(sizeof(int32_t));
  lay->act = take(2 * static_cast<size_t>(m) * L->inter);   // grouped order, padding rows included
  lay->rows = take(sizeof(float) * static_cast<size_t>(total) * L->hidden);
  lay->total = off;
  return STEP_OK;
}

int launched(const char* what) {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? STEP_OK : fail(STEP_EHIP, "%s launch failed: %s", what, hipGetErrorString(e));
}

int align_launch(const int32_t* ids, int total, int E, int bm, int m_max, int32_t* sorted, int32_t* bexp,
                 int32_t* npad, int32_t* brank, hipStream_t s) {
  hipLaunchKernelGGL(gr::k_moe_align, dim3(1), dim3(gr::kMoeAlignThreads), 0, s, ids, total, E, bm, m_max, sorted, bexp,
                     npad, brank);
  return launched("moe align");
}

template <class T>
int forward(const moe_layer* L, char* ws, const MoeLayout& lay, hipStream_t s) {
  const int total = L->n_tokens * L->top_k;
  int32_t* sorted = reinterpret_cast<int32_t*>(ws + lay.sorted);
  int32_t* bexp = reinterpret_cast<int32_t*>(ws + lay.bexp);
  int32_t* npad = reinterpret_cast<int32_t*>(ws + lay.npad);
  int32_t* brank = reinterpret_cast<int32_t*>(ws + lay.brank);
  int rc = align_launch(L->d_expert_ids, total, L->num_experts, MOE_BLOCK_M, lay.m_max, sorted, bexp, npad, brank, s);
  if (rc != STEP_OK) return rc;
  // group blocks in the grid: a multiple of 8, so every XCD gets the same share (the extra blocks
  // lie past the used rows and exit)
  const int mblocks = (lay.m_max / MOE_BLOCK_M + gr::kXcds - 1) / gr::kXcds * gr::kXcds;
  gr::MoeGemmArgs g{};
  g.sorted_ids = sorted;
  g.block_expert = bexp;
  g.num_padded = npad;
  g.block_rank = brank;
  g.total = total;
  g.top_k = L->top_k;
  // gate|up: K = hidden, 8 activation columns per tile, 4 tiles per block
  constexpr int RT = 4;
  g.W = L->d_gate_up;
  g.A = L->d_x;
  g.out = ws + lay.act;
  g.ncols = L->inter;
  g.K = L->hidden;
  // when experts average 32 rows or more, one workgroup takes up to 4 group blocks of an expert
  const bool multi = total >= 32 * L->num_experts;
  g.ntiles = (L->inter + 8 * RT - 1) / (8 * RT);
  const dim3 gu_grid(mblocks * g.ntiles);
  if (multi)
    hipLaunchKernelGGL((gr::k_moe_gemm<T, true, RT, 2, 4>), gu_grid, dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL((gr::k_moe_gemm<T, true, RT, 4, 1>), gu_grid, dim3(256), 0, s, g);
  if ((rc = launched("moe gate|up")) != STEP_OK) return rc;
  // down: K = inter, 16 output columns per tile
  g.W = L->d_down;
  g.A = ws + lay.act;
  g.out = ws + lay.rows;
  g.weights = L->d_weights;
  g.ncols = L->hidden;
  g.K = L->inter;
  g.ntiles = (L->hidden + 16 * RT - 1) / (16 * RT);
  const dim3 dn_grid(mblocks * g.ntiles);
  if (multi)
    hipLaunchKernelGGL((gr::k_moe_gemm<T, false, RT, 2, 4>), dn_grid, dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL((gr::k_moe_gemm<T, false, RT, 2, 1>), dn_grid, dim3(256), 0, s, g);
  if ((rc = launched("moe down")) != STEP_OK) return rc;
  hipLaunchKernelGGL(gr::k_moe_sum<T>, dim3(L->n_tokens, (L->hidden + 1023) / 1024), dim3(256), 0, s,
                     reinterpret_cast<const float*>(ws + lay.rows), L->d_expert_ids, L->top_k, L->num_experts, L->hidden,
                     L->d_out);
  return launched("moe sum");
}

// The allocation-free variant's workspace: one array per GPU, resident from the library's load
// until the process ends. In host code `scratch` names a host-side stand-in, not device memory, so
// its device address is looked up once per device with hipGetSymbolAddress (with that device
// current) and only that address is ever passed to a kernel.
__device__ __align__(256) unsigned char scratch[MOE_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// this device's copy of `scratch` (nullptr and a message on failure)
void* scratch_for_current_device() noexcept {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    fail(STEP_EHIP, "moe_forward_static: hipGetDevice failed: %s", hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    fail(STEP_EUNSUPPORTED, "moe_forward_static: device %d is past the %d devices it keeps a workspace for", dev,
         kMaxDevices);
    return nullptr;
  }
  try {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p) {
        fail(STEP_EHIP, "moe_forward_static: hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
        return nullptr;
      }
      g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
  } catch (...) {
    fail(STEP_EHIP, "moe_forward_static: could not lock the workspace table");
    return nullptr;
  }
}

}  // namespace

extern "C" int32_t moe_align_rows(int32_t total, int32_t num_experts, int32_t block_m) {
  return static_cast<int32_t>(rows_for(total, num_experts, block_m));
}

extern "C" int moe_align(const int32_t* d_expert_ids, int32_t total, int32_t num_experts, int32_t block_m,
                         int32_t* d_sorted_ids, int32_t* d_block_expert, int32_t* d_num_padded, void* stream) {
  // nothing below allocates host memory or throws: the checks are arithmetic and the launch is HIP
  g_err.clear();
  const long long m = rows_for(total, num_experts, block_m);
  if (m < 0) return fail(STEP_EINVAL, "moe_align: total %d, num_experts %d (1..%d), block_m %d (1..65536)", total,
                         num_experts, MOE_MAX_EXPERTS, block_m);
  if ((total > 0 && !d_expert_ids) || !d_sorted_ids || !d_block_expert || !d_num_padded)
    return fail(STEP_EINVAL, "moe_align: NULL device pointer");
  return align_launch(d_expert_ids, total, num_experts, block_m, static_cast<int>(m), d_sorted_ids, d_block_expert,
                      d_num_padded, nullptr, static_cast<hipStream_t>(stream));
}

extern "C" size_t moe_workspace_bytes(const moe_layer* layer) {
  // host arithmetic only; fail() swallows a failed message allocation
  MoeLayout lay;
  if (check_layer(layer, &lay) != STEP_OK) return 0;
  return lay.total;
}

extern "C" int moe_forward(const moe_layer* layer, void* d_workspace, size_t workspace_bytes, void* stream) {
  // as moe_align: checks and launches only, and fail() never throws
  g_err.clear();
  MoeLayout lay;
  int rc = check_layer(layer, &lay);
  if (rc != STEP_OK) return rc;
  if (layer->n_tokens == 0) return STEP_OK;
  if (!layer->d_x || !layer->d_gate_up || !layer->d_down || !layer->d_weights || !layer->d_expert_ids ||
      !layer->d_out || !d_workspace)
    return fail(STEP_EINVAL, "moe_forward: NULL device pointer");
  if (reinterpret_cast<uintptr_t>(d_workspace) % 256)
    return fail(STEP_EINVAL, "moe_forward: workspace must be 256-byte aligned");
  if (workspace_bytes < lay.total)
    return fail(STEP_EINVAL, "moe_forward: workspace %zu bytes, needs %zu", workspace_bytes, lay.total);
  char* ws = static_cast<char*>(d_workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return layer->dtype == STEP_BF16 ? forward<gr::BF16>(layer, ws, lay, s) : forward<gr::F16>(layer, ws, lay, s);
}

extern "C" int moe_forward_static(const moe_layer* layer, void* stream) {
  // as moe_forward, over this device's static workspace: no allocation of any kind
  g_err.clear();
  MoeLayout lay;
  int rc = check_layer(layer, &lay);
  if (rc != STEP_OK) return rc;
  if (lay.total > MOE_STATIC_SCRATCH_BYTES)
    return fail(STEP_EINVAL, "moe_forward_static: the layer needs %zu workspace bytes, the static workspace holds %zu",
                lay.total, static_cast<size_t>(MOE_STATIC_SCRATCH_BYTES));
  if (layer->n_tokens == 0) return STEP_OK;
  if (!layer->d_x || !layer->d_gate_up || !layer->d_down || !layer->d_weights || !layer->d_expert_ids ||
      !layer->d_out)
    return fail(STEP_EINVAL, "moe_forward_static: NULL device pointer");
  char* ws = static_cast<char*>(scratch_for_current_device());
  if (!ws) return STEP_EHIP;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return layer->dtype == STEP_BF16 ? forward<gr::BF16>(layer, ws, lay, s) : forward<gr::F16>(layer, ws, lay, s);
}

extern "C" const char* moe_last_error(void) { return g_err.c_str(); }
