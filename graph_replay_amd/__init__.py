"""Python binding of libstep (include/step.h): one decode / mixed transformer step on an MI355X.

The functions step_workspace_bytes / step_init / step_decode / step_mixed / step_sample /
step_destroy mirror the C ABI one to one and only marshal arguments; every step of the computation
runs in the HIP kernels of libstep.so. ``Decoder`` owns the device memory (allocated with PyTorch)
that the C ABI borrows: the weights with Q|K|V and gate|up stacked once at load time ("Removing
overhead: fusion, graphs and async scheduling", section "Fewer, larger matmuls"), the zero-filled
paged KV pools, the logits / token outputs and the workspace.
"""
from __future__ import annotations

import ctypes as C
from typing import Optional, Sequence

import numpy as np

from . import _lib
from ._lib import (STEP_BF16, STEP_F16, STEP_F32, MoeLayer, StepBatch, StepBuffers, StepConfig, StepPacked,
                   StepWeights)

__all__ = ["Decoder", "StepError", "step_workspace_bytes", "step_init", "step_decode", "step_mixed", "step_sample",
           "step_destroy", "step_set_device_status", "step_attention_slots", "load", "moe_align_rows", "moe_align", "moe_workspace_bytes", "moe_forward", "moe_forward_static",
           "MoeLayer"]

load = _lib.load


class StepError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libstep error {code}: {msg}")
        self.code = code


def _raise(rc: int, ctx) -> None:
    if rc == _lib.STEP_OK:
        return
    msg = _lib.load().step_last_error(ctx).decode() if ctx else ""
    if rc == _lib.STEP_EINVAL:
        raise ValueError(msg)
    raise StepError(rc, msg)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _ip(a: Optional[np.ndarray]):
    return a.ctypes.data_as(_lib.I32P) if a is not None else None


def _fp(a: Optional[np.ndarray]):
    return a.ctypes.data_as(_lib.F32P) if a is not None else None


# ------------------------------------------------------------------------------------------ C ABI

def step_workspace_bytes(cfg: StepConfig) -> int:
    return int(_lib.load().step_workspace_bytes(C.byref(cfg)))


def step_init(cfg: StepConfig, weights: StepWeights, buffers: StepBuffers, stream: int) -> C.c_void_p:
    ctx = C.c_void_p()
    rc = _lib.load().step_init(C.byref(cfg), C.byref(weights), C.byref(buffers), C.c_void_p(stream), C.byref(ctx))
    if rc != _lib.STEP_OK:
        msg = _lib.load().step_last_error(ctx).decode() if ctx else ""
        if ctx:
            _lib.load().step_destroy(ctx)
        _raise_msg(rc, msg)
    return ctx


def _raise_msg(rc: int, msg: str):
    if rc == _lib.STEP_EINVAL:
        raise ValueError(msg)
    raise StepError(rc, msg)


def step_decode(ctx, batch: Optional[StepBatch]) -> None:
    _raise(_lib.load().step_decode(ctx, C.byref(batch) if batch is not None else None), ctx)


def step_mixed(ctx, packed: StepPacked) -> None:
    _raise(_lib.load().step_mixed(ctx, C.byref(packed)), ctx)


def step_sample(ctx, d_logits: int, rows: int, ld: int, vocab: int, h_temperature: Optional[np.ndarray],
                h_top_k: Optional[np.ndarray], h_top_p: Optional[np.ndarray], d_uniforms: Optional[int], seed: int,
                counter: int, d_tokens: int) -> None:
    t = _f32(h_temperature) if h_temperature is not None else None
    k = _i32(h_top_k) if h_top_k is not None else None
    p = _f32(h_top_p) if h_top_p is not None else None
    rc = _lib.load().step_sample(ctx, C.cast(C.c_void_p(d_logits), _lib.F32P), rows, ld, vocab, _fp(t), _ip(k), _fp(p),
                                 C.cast(C.c_void_p(d_uniforms), _lib.F32P) if d_uniforms else None,
                                 C.c_uint64(seed), C.c_uint64(counter), C.cast(C.c_void_p(d_tokens), _lib.I32P))
    _raise(rc, ctx)


def step_device_status(ctx) -> None:
    _raise(_lib.load().step_device_status(ctx), ctx)


def step_set_device_status(ctx, site: int) -> None:
    _raise(_lib.load().step_set_device_status(ctx, site), ctx)


def step_attention_slots(cfg: StepConfig, rows: int, max_len: int):
    """(partial slots one attention launch uses, partial slots the workspace holds); host only."""
    cap = C.c_int64(-1)
    n = int(_lib.load().step_attention_slots(C.byref(cfg), rows, max_len, C.byref(cap)))
    return n, int(cap.value)


def step_destroy(ctx) -> None:
    if ctx:
        _lib.load().step_destroy(ctx)


# -------------------------------------------------------------------------------- MoE layer (moe.h)

def _moe_raise(rc: int) -> None:
    if rc == _lib.STEP_OK:
        return
    msg = _lib.load().moe_last_error().decode()
    if rc == _lib.STEP_EINVAL:
        raise ValueError(msg)
    raise StepError(rc, msg)


def moe_align_rows(total: int, num_experts: int, block_m: int) -> int:
    """Rows of the grouped layout (-1 when the sizes are out of range)."""
    return int(_lib.load().moe_align_rows(total, num_experts, block_m))


def _check_dev(name, t, dtype, torch):
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} CUDA tensor")


def moe_align(expert_ids, num_experts: int, block_m: int):
    """expert_ids: int32 CUDA tensor [N, k] (or flat). Returns (sorted_ids, block_expert, num_padded)
    int32 CUDA tensors, enqueued on the current stream."""
    import torch
    _check_dev("expert_ids", expert_ids, torch.int32, torch)
    total = expert_ids.numel()
    rows = moe_align_rows(total, num_experts, block_m)
    if rows < 0:
        raise ValueError(f"moe_align: sizes out of range (total {total}, experts {num_experts}, block_m {block_m})")
    dev = expert_ids.device
    sorted_ids = torch.empty(rows, dtype=torch.int32, device=dev)
    block_expert = torch.empty(rows // block_m, dtype=torch.int32, device=dev)
    num_padded = torch.empty(1, dtype=torch.int32, device=dev)
    ip = lambda t: C.cast(C.c_void_p(t.data_ptr()), _lib.I32P)
    _moe_raise(_lib.load().moe_align(ip(expert_ids), total, num_experts, block_m, ip(sorted_ids), ip(block_expert),
                                     ip(num_padded), C.c_void_p(torch.cuda.current_stream(dev).cuda_stream)))
    return sorted_ids, block_expert, num_padded


def _moe_struct(x, gate_up, down, weights, expert_ids, out):
    import torch
    code = {torch.bfloat16: STEP_BF16, torch.float16: STEP_F16}.get(x.dtype)
    if code is None:
        raise ValueError("moe_forward: x must be bfloat16 or float16")
    for name, t in (("x", x), ("gate_up", gate_up), ("down", down), ("out", out)):
        _check_dev(name, t, x.dtype, torch)
    _check_dev("weights", weights, torch.float32, torch)
    _check_dev("expert_ids", expert_ids, torch.int32, torch)
    n, d = x.shape
    E, two_i, d2 = gate_up.shape
    if d2 != d or tuple(down.shape) != (E, d, two_i // 2) or expert_ids.dim() != 2 or expert_ids.shape[0] != n \
            or tuple(weights.shape) != tuple(expert_ids.shape) or tuple(out.shape) != (n, d) or two_i % 2:
        raise ValueError("moe_forward: shapes must be x [N, D], gate_up [E, 2I, D], down [E, D, I], "
                         "weights / expert_ids [N, k], out [N, D]")
    return MoeLayer(dtype=code, n_tokens=n, top_k=expert_ids.shape[1], num_experts=E, hidden=d, inter=two_i // 2,
                    d_x=x.data_ptr(), d_gate_up=gate_up.data_ptr(), d_down=down.data_ptr(),
                    d_weights=C.cast(C.c_void_p(weights.data_ptr()), _lib.F32P),
                    d_expert_ids=C.cast(C.c_void_p(expert_ids.data_ptr()), _lib.I32P), d_out=out.data_ptr())


def moe_workspace_bytes(x, gate_up, down, weights, expert_ids, out) -> int:
    return int(_lib.load().moe_workspace_bytes(C.byref(_moe_struct(x, gate_up, down, weights, expert_ids, out))))


def moe_forward(x, gate_up, down, weights, expert_ids, out=None, workspace=None):
    """The MoE MLP layer through libstep's moe_forward on the current stream. out [N, D] and the
    uint8 workspace are allocated here when not given (pass both for graph capture)."""
    import torch
    if out is None:
        out = torch.empty_like(x)
    L = _moe_struct(x, gate_up, down, weights, expert_ids, out)
    lib = _lib.load()
    need = int(lib.moe_workspace_bytes(C.byref(L)))
    if need == 0:
        _moe_raise(lib.moe_forward(C.byref(L), None, 0, None))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    if workspace.numel() < need:
        raise ValueError(f"moe_forward: workspace of {workspace.numel()} bytes, needs {need}")
    _moe_raise(lib.moe_forward(C.byref(L), C.c_void_p(workspace.data_ptr()), workspace.numel(),
                               C.c_void_p(torch.cuda.current_stream(x.device).cuda_stream)))
    return out


def moe_forward_static(x, gate_up, down, weights, expert_ids, out):
    """moe_forward over libstep's static per-device workspace (no workspace argument, nothing
    allocated by the call); out [N, D] must be given."""
    import torch
    L = _moe_struct(x, gate_up, down, weights, expert_ids, out)
    _moe_raise(_lib.load().moe_forward_static(C.byref(L), C.c_void_p(torch.cuda.current_stream(x.device).cuda_stream)))
    return out


# ------------------------------------------------------------------------------------------ owner

_DTYPE_CODE = {"f32": STEP_F32, "bf16": STEP_BF16, "f16": STEP_F16}


class Decoder:
    """Device buffers + libstep context for one model.

    ``weights`` holds CPU (or device) tensors in the storage dtype with the names of
    ``synth.make_weights``: embed, lm_head, final_norm and per layer in_norm, wq, wk, wv, bq, bk, bv,
    q_norm, k_norm, wo, post_norm, wg, wu, wd (row-major [out, in]).
    """

    def __init__(self, shape, weights: dict, *, num_blocks: int, max_blocks_per_seq: int, max_position: int,
                 max_batch: int = 1, buckets: Optional[Sequence[int]] = None, max_tokens: int = 0,
                 max_reqs: int = 0, max_logit_rows: int = 0, use_graphs: bool = True, history: bool = False,
                 mixed_buckets: Optional[Sequence[int]] = None, sampling_filters: bool = False,
                 weight_prefetch: bool = True, persistent_decode: bool = False,
                 balanced_attention_rows: int = 0, device: str = "cuda:0"):
        import torch
        lib = _lib.load()
        self.torch = torch
        self.shape = shape
        self.device = torch.device(device)
        dt = shape.torch_dtype
        dev = self.device
        self._keep = []

        def up(t):
            if t is None:
                return None
            x = t.to(device=dev, dtype=dt).contiguous()
            self._keep.append(x)
            return x

        embed = up(weights["embed"])
        lm_head = embed if weights["lm_head"] is weights["embed"] else up(weights["lm_head"])
        final_norm = up(weights["final_norm"])
        names = ("in_norm", "qkv_w", "qkv_b", "q_norm", "k_norm", "o_w", "post_norm", "gate_up_w", "down_w")
        per = {n: [] for n in names}
        for lw in weights["layers"]:
            per["in_norm"].append(up(lw["in_norm"]))
            per["qkv_w"].append(up(torch.cat([lw["wq"], lw["wk"], lw["wv"]], 0)))
            per["qkv_b"].append(up(torch.cat([lw["bq"], lw["bk"], lw["bv"]], 0)) if shape.qkv_bias else None)
            per["q_norm"].append(up(lw["q_norm"]) if shape.qk_norm else None)
            per["k_norm"].append(up(lw["k_norm"]) if shape.qk_norm else None)
            per["o_w"].append(up(lw["wo"]))
            per["post_norm"].append(up(lw["post_norm"]))
            per["gate_up_w"].append(up(torch.cat([lw["wg"], lw["wu"]], 0)))
            per["down_w"].append(up(lw["wd"]))
        L = shape.layers
        self._ptr_arrays = {}

        def parr(ts):
            a = (C.c_void_p * L)(*[t.data_ptr() if t is not None else None for t in ts])
            self._ptr_arrays[id(a)] = a
            return C.cast(a, _lib.PP)

        w = StepWeights()
        w.d_embed, w.d_lm_head, w.d_final_norm = embed.data_ptr(), lm_head.data_ptr(), final_norm.data_ptr()
        for n in names:
            has = all(t is not None for t in per[n])
            setattr(w, "d_" + n, parr(per[n]) if has else None)
        self.weights_struct = w

        # KV pools, zero-filled, per layer: K [num_blocks][kv_heads][16][head_dim] (key-major) and
        # V [num_blocks][kv_heads][head_dim][16] (dim-major)
        k_shape = (num_blocks, shape.kv_heads, 16, shape.head_dim)
        v_shape = (num_blocks, shape.kv_heads, shape.head_dim, 16)
        self.k_pool = [torch.zeros(k_shape, dtype=dt, device=dev) for _ in range(L)]
        self.v_pool = [torch.zeros(v_shape, dtype=dt, device=dev) for _ in range(L)]
        rows = max(max_batch, max_logit_rows)
        self.logits = torch.zeros((rows, shape.vocab), dtype=torch.float32, device=dev)
        self.tokens = torch.zeros(rows, dtype=torch.int32, device=dev)
        self.history = (torch.full((max_batch, max_position), -1, dtype=torch.int32, device=dev)
                        if history else None)

        cfg = StepConfig()
        cfg.dtype = _DTYPE_CODE[shape.dtype]
        cfg.layers, cfg.hidden, cfg.q_heads, cfg.kv_heads = L, shape.hidden, shape.q_heads, shape.kv_heads
        cfg.head_dim, cfg.intermediate, cfg.vocab = shape.head_dim, shape.intermediate, shape.vocab
        cfg.qk_norm, cfg.qkv_bias = int(shape.qk_norm), int(shape.qkv_bias)
        cfg.rms_eps, cfg.rope_theta = shape.eps, shape.theta
        cfg.block_size, cfg.num_blocks, cfg.max_blocks_per_seq = 16, num_blocks, max_blocks_per_seq
        cfg.max_position, cfg.max_batch = max_position, max_batch
        cfg.max_tokens, cfg.max_reqs, cfg.max_logit_rows = max_tokens, max_reqs, max_logit_rows
        buckets = list(buckets) if buckets else [max_batch]
        if len(buckets) > _lib.MAX_BUCKETS:
            raise ValueError("too many buckets")
        cfg.num_buckets = len(buckets)
        for i, b in enumerate(buckets):
            cfg.buckets[i] = int(b)
        cfg.use_graphs = int(use_graphs)
        mixed_buckets = list(mixed_buckets) if mixed_buckets else []
        if len(mixed_buckets) > _lib.MAX_BUCKETS:
            raise ValueError("too many mixed buckets")
        cfg.num_mixed_buckets = len(mixed_buckets)
        for i, b in enumerate(mixed_buckets):
            cfg.mixed_buckets[i] = int(b)
        cfg.sampling_filters = int(sampling_filters)
        cfg.weight_prefetch = int(weight_prefetch)
        cfg.persistent_decode = int(persistent_decode)
        cfg.balanced_attention_rows = int(balanced_attention_rows)
        self.cfg = cfg
        self.buckets = buckets
        nbytes = step_workspace_bytes(cfg)
        if nbytes == 0:
            raise ValueError("invalid configuration")
        self.workspace = torch.empty(nbytes + 256, dtype=torch.uint8, device=dev)
        ws_ptr = (self.workspace.data_ptr() + 255) // 256 * 256

        b = StepBuffers()
        self._kp = (C.c_void_p * L)(*[t.data_ptr() for t in self.k_pool])
        self._vp = (C.c_void_p * L)(*[t.data_ptr() for t in self.v_pool])
        b.d_k_pool, b.d_v_pool = C.cast(self._kp, _lib.PP), C.cast(self._vp, _lib.PP)
        b.d_logits = C.cast(C.c_void_p(self.logits.data_ptr()), _lib.F32P)
        b.d_tokens = C.cast(C.c_void_p(self.tokens.data_ptr()), _lib.I32P)
        b.d_history = C.cast(C.c_void_p(self.history.data_ptr()), _lib.I32P) if history else None
        b.d_workspace, b.workspace_bytes = ws_ptr, nbytes
        self.buffers_struct = b
        torch.cuda.synchronize(dev)
        self.stream = torch.cuda.current_stream(dev)
        self.ctx = step_init(cfg, w, b, self.stream.cuda_stream)

    # -- steps
    def decode(self, tokens, positions, seq_lens, slots, block_table, temperature=None, seed: int = 0,
               top_k=None, top_p=None) -> None:
        t, p, s, sl = _i32(tokens), _i32(positions), _i32(seq_lens), _i32(slots)
        bt = _i32(block_table)
        if bt.ndim != 2 or bt.shape[0] != t.shape[0]:
            raise ValueError("block_table must be [rows, width]")
        temp = _f32(temperature) if temperature is not None else None
        tk = _i32(top_k) if top_k is not None else None
        tp = _f32(top_p) if top_p is not None else None
        hb = StepBatch(num_rows=t.shape[0], bt_width=bt.shape[1], h_tokens=_ip(t), h_positions=_ip(p),
                       h_seq_lens=_ip(s), h_slot_mapping=_ip(sl), h_block_table=_ip(bt), h_temperature=_fp(temp),
                       seed=seed, h_top_k=_ip(tk), h_top_p=_fp(tp))
        step_decode(self.ctx, hb)

    def decode_continue(self) -> None:
        step_decode(self.ctx, None)

    def mixed(self, query_start_loc, seq_lens, tokens, positions, slots, block_table, logits_indices,
              num_prefill_reqs: int, temperature=None, seed: int = 0, prefill_attention: int = 0, top_k=None,
              top_p=None) -> None:
        qsl, sl_, t, p, s = _i32(query_start_loc), _i32(seq_lens), _i32(tokens), _i32(positions), _i32(slots)
        bt, li = _i32(block_table), _i32(logits_indices)
        temp = _f32(temperature) if temperature is not None else None
        nreq = qsl.shape[0] - 1
        hp = StepPacked(num_tokens=t.shape[0], num_prefill_reqs=num_prefill_reqs,
                        num_decode_reqs=nreq - num_prefill_reqs, num_logits=li.shape[0], bt_width=bt.shape[1],
                        h_query_start_loc=_ip(qsl), h_seq_lens=_ip(sl_), h_tokens=_ip(t), h_positions=_ip(p),
                        h_slot_mapping=_ip(s), h_block_table=_ip(bt), h_logits_indices=_ip(li),
                        h_temperature=_fp(temp), seed=seed, prefill_attention=prefill_attention)
        tk = _i32(top_k) if top_k is not None else None
        tp = _f32(top_p) if top_p is not None else None
        hp.h_top_k, hp.h_top_p = _ip(tk), _fp(tp)
        step_mixed(self.ctx, hp)

    def sample(self, logits, temperature=None, uniforms=None, seed: int = 0, counter: int = 0, top_k=None,
               top_p=None):
        torch = self.torch
        rows, ld = logits.shape
        out = torch.empty(rows, dtype=torch.int32, device=self.device)
        step_sample(self.ctx, logits.data_ptr(), rows, ld, ld, temperature, top_k, top_p,
                    uniforms.data_ptr() if uniforms is not None else None, seed, counter, out.data_ptr())
        return out

    def profile_decode(self, max_kernels: int = 4096):
        """One eager, event-timed decode step (advances the state). Returns [(kind name, ms), ...]."""
        lib = _lib.load()
        ms = np.zeros(max_kernels, np.float32)
        kind = np.zeros(max_kernels, np.int32)
        n = lib.step_profile_decode(self.ctx, max_kernels, _fp(ms), _ip(kind))
        if n < 0:
            _raise(n, self.ctx)
        n = min(n, max_kernels)
        return [(lib.step_kernel_kind_name(int(kind[i])).decode(), float(ms[i])) for i in range(n)]

    def device_status(self) -> None:
        """Raise StepError if a wait inside a persistent decode step gave up (waits for the stream)."""
        step_device_status(self.ctx)

    def set_device_status(self, site: int) -> None:
        """Set the persistent step's give-up flag as a wait that gave up at `site` would (tests)."""
        step_set_device_status(self.ctx, site)

    def phase_stamps(self):
        """Phase timestamps (us) of the last profiled persistent step, or None."""
        lib = _lib.load()
        buf = (C.c_double * 512)()
        n = lib.step_phase_stamps(self.ctx, 512, buf)
        if n < 0:
            _raise(n, self.ctx)
        return [buf[i] for i in range(min(n, 512))] if n > 0 else None

    def last_bucket(self) -> int:
        return int(_lib.load().step_last_bucket(self.ctx))

    def kernels_per_decode(self, bucket: int) -> int:
        return int(_lib.load().step_kernels_per_decode(self.ctx, bucket))

    def last_mixed_bucket(self) -> int:
        return int(_lib.load().step_last_mixed_bucket(self.ctx))

    def close(self) -> None:
        if getattr(self, "ctx", None):
            step_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
