"""ctypes declarations of libstep's C ABI (include/step.h, include/moe.h). Argument marshalling only."""
import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libstep.so")

STEP_OK, STEP_EINVAL, STEP_EUNSUPPORTED, STEP_EHIP, STEP_ECAPTURE, STEP_ESTATE = 0, -1, -2, -3, -4, -5
STEP_F32, STEP_BF16, STEP_F16 = 0, 1, 2
MAX_BUCKETS = 16

P = C.c_void_p
PP = C.POINTER(C.c_void_p)
I32P = C.POINTER(C.c_int32)
F32P = C.POINTER(C.c_float)


class StepConfig(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("dtype", "layers", "hidden", "q_heads", "kv_heads", "head_dim",
                                         "intermediate", "vocab", "qk_norm", "qkv_bias")] + [
        ("rms_eps", C.c_float), ("rope_theta", C.c_float)] + [
        (n, C.c_int32) for n in ("block_size", "num_blocks", "max_blocks_per_seq", "max_position", "max_batch",
                                 "max_tokens", "max_reqs", "max_logit_rows", "num_buckets")] + [
        ("buckets", C.c_int32 * MAX_BUCKETS), ("use_graphs", C.c_int32),
        ("num_mixed_buckets", C.c_int32), ("mixed_buckets", C.c_int32 * MAX_BUCKETS),
        ("sampling_filters", C.c_int32),
        ("weight_prefetch", C.c_int32),
        ("persistent_decode", C.c_int32),
        ("balanced_attention_rows", C.c_int32)]


class StepWeights(C.Structure):
    _fields_ = [("d_embed", P), ("d_lm_head", P), ("d_final_norm", P)] + [
        (n, PP) for n in ("d_in_norm", "d_qkv_w", "d_qkv_b", "d_q_norm", "d_k_norm", "d_o_w", "d_post_norm",
                          "d_gate_up_w", "d_down_w")]


class StepBuffers(C.Structure):
    _fields_ = [("d_k_pool", PP), ("d_v_pool", PP), ("d_logits", F32P), ("d_tokens", I32P), ("d_history", I32P),
                ("d_workspace", P), ("workspace_bytes", C.c_size_t)]


class StepBatch(C.Structure):
    _fields_ = [("num_rows", C.c_int32), ("bt_width", C.c_int32), ("h_tokens", I32P), ("h_positions", I32P),
                ("h_seq_lens", I32P), ("h_slot_mapping", I32P), ("h_block_table", I32P), ("h_temperature", F32P),
                ("seed", C.c_uint64), ("h_top_k", I32P), ("h_top_p", F32P)]


class StepPacked(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("num_tokens", "num_prefill_reqs", "num_decode_reqs", "num_logits",
                                         "bt_width")] + [
        (n, I32P) for n in ("h_query_start_loc", "h_seq_lens", "h_tokens", "h_positions", "h_slot_mapping",
                            "h_block_table", "h_logits_indices")] + [
        ("h_temperature", F32P), ("seed", C.c_uint64), ("prefill_attention", C.c_int32),
        ("h_top_k", I32P), ("h_top_p", F32P)]


class MoeLayer(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("dtype", "n_tokens", "top_k", "num_experts", "hidden", "inter")] + [
        ("d_x", P), ("d_gate_up", P), ("d_down", P), ("d_weights", F32P), ("d_expert_ids", I32P), ("d_out", P)]


EXPORTS = {
    "step_workspace_bytes": (C.c_size_t, [C.POINTER(StepConfig)]),
    "step_init": (C.c_int, [C.POINTER(StepConfig), C.POINTER(StepWeights), C.POINTER(StepBuffers), P,
                            C.POINTER(P)]),
    "step_decode": (C.c_int, [P, C.POINTER(StepBatch)]),
    "step_mixed": (C.c_int, [P, C.POINTER(StepPacked)]),
    "step_sample": (C.c_int, [P, F32P, C.c_int32, C.c_int32, C.c_int32, F32P, I32P, F32P, F32P, C.c_uint64,
                              C.c_uint64, I32P]),
    "step_profile_decode": (C.c_int, [P, C.c_int32, F32P, I32P]),
    "step_kernel_kind_name": (C.c_char_p, [C.c_int32]),
    "step_last_bucket": (C.c_int, [P]),
    "step_kernels_per_decode": (C.c_int, [P, C.c_int32]),
    "step_last_mixed_bucket": (C.c_int, [P]),
    "step_last_error": (C.c_char_p, [P]),
    "step_device_status": (C.c_int, [P]),
    "step_phase_stamps": (C.c_int, [P, C.c_int32, C.POINTER(C.c_double)]),
    "step_set_device_status": (C.c_int, [P, C.c_int32]),
    "step_attention_slots": (C.c_int32, [C.POINTER(StepConfig), C.c_int32, C.c_int32, C.POINTER(C.c_int64)]),
    "step_destroy": (None, [P]),
    "moe_align_rows": (C.c_int32, [C.c_int32, C.c_int32, C.c_int32]),
    "moe_align": (C.c_int, [I32P, C.c_int32, C.c_int32, C.c_int32, I32P, I32P, I32P, P]),
    "moe_workspace_bytes": (C.c_size_t, [C.POINTER(MoeLayer)]),
    "moe_forward": (C.c_int, [C.POINTER(MoeLayer), P, C.c_size_t, P]),
    "moe_forward_static": (C.c_int, [C.POINTER(MoeLayer), P]),
    "moe_last_error": (C.c_char_p, []),
}

_lib = None


def load(path: str = LIB_PATH):
    """Load libstep.so; raise if it is not built (there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libstep.so not found at {path}: build it with graph_replay_amd/build.py "
                           "(or __graft_entry__.build()); there is no CPU fallback")
    lib = C.CDLL(path)
    for name, (res, args) in EXPORTS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
