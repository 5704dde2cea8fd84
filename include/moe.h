/* moe.h - C ABI of libstep's mixture-of-experts layer: the expert grouping and the grouped-GEMM
 * expert MLP, on one AMD Instinct MI355X (gfx950), with no host read of any routing value.
 *
 * The method is "Removing overhead: fusion, graphs and async scheduling", section "A MoE layer
 * that never asks the host": the N * k (token, slot) assignments are grouped by expert, each group
 * padded to a multiple of BLOCK_M rows, in device work whose shapes depend only on N, k, E and
 * BLOCK_M; then one launch per projection multiplies each BLOCK_M-row block by its expert's
 * weights (the first reading token rows, the second the rows of the first), and each token sums
 * its k rows, scaled by their router weights.
 *
 * Conventions are those of step.h: d_* pointers are DEVICE memory owned by the caller, calls only
 * enqueue work on the given stream (a hipStream_t; NULL is the default stream) and are graph-
 * capturable, return STEP_OK or a negative STEP_E* code and never throw. The message of the last
 * error on the calling thread is in moe_last_error(). No call allocates device memory.
 */
#ifndef GRAPH_REPLAY_AMD_MOE_H
#define GRAPH_REPLAY_AMD_MOE_H

#include <stddef.h>
#include <stdint.h>

#include "step.h"

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_BLOCK_M 16        /* group block rows of moe_forward's grouped GEMMs */
#define MOE_MAX_EXPERTS 1024

/* Rows of the grouped layout for `total` assignments: total + E * (block_m - 1) rounded up to a
 * multiple of block_m (every group padded by at most block_m - 1 rows). Returns -1 when an
 * argument is out of range (total < 0, E not in [1, MOE_MAX_EXPERTS], block_m not in [1, 65536])
 * or the count does not fit an int32. */
int32_t moe_align_rows(int32_t total, int32_t num_experts, int32_t block_m);

/* Group the assignments by expert (the page's moe_align).
 *   d_expert_ids   [total] int32, assignment i = token * k + slot; ids outside [0, E) belong
 *                  to no group (they get no row).
 *   d_sorted_ids   [moe_align_rows(total, E, block_m)] int32 out: row r of the grouped layout holds
 *                  the assignment it computes, or `total` for a padding row. Expert e's group
 *                  (groups in expert order from row 0) lists its assignments in increasing order,
 *                  then padding up to a multiple of block_m.
 *   d_block_expert [rows / block_m] int32 out: the expert of each block_m-row block; blocks at or
 *                  past num_padded hold E - 1.
 *   d_num_padded   [1] int32 out: rows used by the groups (a multiple of block_m).
 * Results are exact and independent of thread timing. STEP_EINVAL for bad sizes or a NULL pointer
 * that is needed (d_expert_ids may be NULL only when total == 0). */
int moe_align(const int32_t* d_expert_ids, int32_t total, int32_t num_experts, int32_t block_m,
              int32_t* d_sorted_ids, int32_t* d_block_expert, int32_t* d_num_padded, void* stream);

typedef struct {
  int32_t dtype;        /* STEP_BF16 or STEP_F16: x, the weights and out */
  int32_t n_tokens;     /* N >= 0 */
  int32_t top_k;        /* k >= 1 experts per token */
  int32_t num_experts;  /* E in [1, MOE_MAX_EXPERTS] */
  int32_t hidden;       /* D, a positive multiple of 32 */
  int32_t inter;        /* I (expert width), a positive multiple of 32 */
  const void* d_x;            /* [N][D] token rows */
  const void* d_gate_up;      /* [E][2I][D]: rows 0..I-1 the gate, rows I..2I-1 the up projection */
  const void* d_down;         /* [E][D][I] */
  const float* d_weights;     /* [N][k] router weights, fp32 */
  const int32_t* d_expert_ids;/* [N][k] expert of each slot (ids outside [0, E) add nothing) */
  void* d_out;                /* [N][D] out: sum over j of w[t][j] * down_e (silu(g) * u) */
} moe_layer;

/* Workspace bytes moe_forward needs for this layer (0 when the sizes are invalid): the grouping
 * (sorted ids, block experts, block ranks, row count), the activation rows in grouped order
 * [moe_align_rows(N * k, E, MOE_BLOCK_M)][I] in the dtype and the weighted down rows [N * k][D]
 * in fp32. */
size_t moe_workspace_bytes(const moe_layer* layer);

/* The MoE MLP layer: grouping, gate|up grouped GEMM with SiLU(gate) * up in its epilogue, down
 * grouped GEMM scaled by the router weight, and the per-token sum of the k rows in slot order
 * (fp32, rounded once to the dtype). Four kernel launches, no host read of device data, so the
 * call can be captured into a graph; the grouped GEMMs' grids are sized for the worst case and
 * their blocks past the used rows exit at once. d_workspace must hold moe_workspace_bytes and
 * be 256-byte aligned; it must not be shared with a call in flight. STEP_EINVAL for bad sizes or
 * pointers, STEP_EUNSUPPORTED for another dtype, STEP_EHIP when a launch fails. */
int moe_forward(const moe_layer* layer, void* d_workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of moe_forward_static's static per-device workspace (16 MiB): enough for
 * moe_workspace_bytes at decode-size batches, e.g. up to 177 tokens at the Qwen3-30B-A3B expert
 * shape (128 experts, top 8, hidden 2048, expert width 768). */
#define MOE_STATIC_SCRATCH_BYTES (16u << 20)

/* moe_forward without a caller workspace, for callers that cannot allocate (code under graph
 * capture, tight serving loops, harnesses that forbid allocation): the same four launches and the
 * same results, over a workspace of MOE_STATIC_SCRATCH_BYTES that the library holds on each GPU
 * from its load until the process ends (its device address is looked up once per device, on the
 * first call made with that device current). The call allocates nothing, device or host.
 * STEP_EINVAL when moe_workspace_bytes(layer) exceeds MOE_STATIC_SCRATCH_BYTES (no launch is
 * made), and the errors of moe_forward otherwise. Every call on one GPU shares that GPU's
 * workspace, and each call rewrites all of it that it reads, so nothing has to be cleared between
 * calls; calls that overlap on one GPU (on different streams, or on one stream under different
 * graphs replayed concurrently) race and must not be issued. */
int moe_forward_static(const moe_layer* layer, void* stream);

/* Message of the last error on this thread ("" when none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif
