"""ctypes binding of libbci (include/bci.h).  Argument marshalling only.

Each ``bci_*`` function here has the name and argument order of the C entry
point.  Tensor arguments may be torch tensors (their device pointer is
passed), raw integer addresses or None (NULL).  Streams may be a
torch.cuda.Stream, an integer hipStream_t or None (torch's current stream).
A non-zero status raises BciError with the library's last-error text; there
is no fallback of any kind: if libbci.so is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbci.so")

BCI_OK, BCI_E_INVALID, BCI_E_UNSUPPORTED, BCI_E_HIP, BCI_E_WORKSPACE, BCI_E_STATE = 0, -1, -2, -3, -4, -5
BCI_MODE_INVARIANT, BCI_MODE_FAST = 0, 1
BCI_KV_BF16, BCI_KV_FP8_E4M3 = 0, 1
BCI_EPI_BF16, BCI_EPI_F32, BCI_EPI_SILU_MUL = 0, 1, 2
STATUS_NAMES = {0: "BCI_OK", -1: "BCI_E_INVALID", -2: "BCI_E_UNSUPPORTED", -3: "BCI_E_HIP",
                -4: "BCI_E_WORKSPACE", -5: "BCI_E_STATE"}

# every symbol the header declares (checked by the CPU test suite)
EXPORTS = [
    "bci_create", "bci_destroy", "bci_last_error", "bci_workspace_bytes", "bci_bind_weights",
    "bci_weight_version", "bci_bind_kv_cache", "bci_set_batch", "bci_forward_logprobs",
    "bci_op_embed", "bci_op_add_rmsnorm", "bci_op_gemm_bf16", "bci_op_rope_kv_write",
    "bci_op_kv_gather_dequant", "bci_op_attention", "bci_op_gather_scored",
    "bci_op_lmhead_logprob", "bci_op_moe_topk", "bci_op_gemm_bf16_ksplit", "bci_op_moe_forward", "bci_profile_begin",
    "bci_profile_end", "bci_forward_logprobs_graph", "bci_graph_count", "bci_graph_reset",
    "bci_op_index_key_write", "bci_op_index_scores", "bci_op_sparse_topk",
    "bci_op_sparse_attention", "bci_ssd_create", "bci_ssd_destroy", "bci_ssd_last_error",
    "bci_ssd_slot_bytes", "bci_ssd_set_batch", "bci_ssd_forward", "bci_op_transpose_bf16",
    "bci_op_add_rmsnorm_backward", "bci_op_silu_mul_backward", "bci_op_logprob_backward_dz",
    "bci_op_rope_backward",
    "bci_op_attention_backward", "bci_lmhead_logprob_noalloc", "bci_measure_mfma_rate",
]


class BciError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class ModelConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim", "intermediate", "vocab")] + \
               [("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float)] + \
               [(n, ctypes.c_int32) for n in
                ("kv_dtype", "kv_block_tokens", "attn_segment_keys", "max_tokens_per_call",
                 "max_seqs_per_call", "max_scored_per_call", "max_position", "mode",
                 "n_experts", "top_k", "expert_intermediate", "n_shared_experts",
                 "attn_split_mode")]


_P32 = ctypes.POINTER(ctypes.c_int32)


class SsdConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("n_heads", "head_dim", "d_state", "n_groups", "max_tokens_per_call",
                 "max_seqs_per_call")]


class Batch(ctypes.Structure):
    _fields_ = [("n_seqs", ctypes.c_int32), ("n_tokens", ctypes.c_int32),
                ("n_scored", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("tokens", _P32), ("cu_q", _P32), ("pos0", _P32), ("block_table", _P32),
                ("score_rows", _P32), ("score_ids", _P32)]


_lib = None


def load() -> ctypes.CDLL:
    """Load libbci.so (built in-tree by bitwise_consistent_rl_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m bitwise_consistent_rl_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, st = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32
    sig = {
        "bci_create": (st, [ctypes.POINTER(ModelConfig), i32, ctypes.POINTER(vp)]),
        "bci_destroy": (None, [vp]),
        "bci_last_error": (ctypes.c_char_p, [vp]),
        "bci_workspace_bytes": (ctypes.c_uint64, [vp]),
        "bci_bind_weights": (st, [vp, ctypes.POINTER(vp), i32, ctypes.c_uint64]),
        "bci_weight_version": (ctypes.c_uint64, [vp]),
        "bci_bind_kv_cache": (st, [vp, vp, vp, vp, vp, i32]),
        "bci_set_batch": (st, [vp, ctypes.POINTER(Batch), vp]),
        "bci_forward_logprobs": (st, [vp, vp, vp]),
        "bci_forward_logprobs_graph": (st, [vp, vp, vp]),
        "bci_graph_count": (i32, [vp]),
        "bci_graph_reset": (st, [vp]),
        "bci_op_embed": (st, [vp, vp, vp, vp]),
        "bci_op_add_rmsnorm": (st, [vp, vp, vp, vp, vp, i32, i32, ctypes.c_float, vp]),
        "bci_op_gemm_bf16": (st, [vp, vp, vp, vp, i32, i32, i32, i32, vp]),
        "bci_op_gemm_bf16_ksplit": (st, [vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp]),
        "bci_op_rope_kv_write": (st, [vp, vp, vp, i32, vp]),
        "bci_op_kv_gather_dequant": (st, [vp, i32, i32, i32, vp, vp, vp]),
        "bci_op_attention": (st, [vp, vp, i32, vp, vp]),
        "bci_op_gather_scored": (st, [vp, vp, i32, vp, vp]),
        "bci_op_lmhead_logprob": (st, [vp, vp, vp, vp, i32, i32, i32, vp, vp]),
        "bci_lmhead_logprob_noalloc": (st, [vp, vp, vp, i32, i32, i32, vp, vp]),
        "bci_op_moe_topk": (st, [vp, vp, i32, vp, vp, vp]),
        "bci_op_moe_forward": (st, [vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp]),
        "bci_op_index_key_write": (st, [vp, vp, i32, vp, vp, i32, vp]),
        "bci_op_index_scores": (st, [vp, vp, vp, i32, i32, vp, vp, i32, vp, ctypes.c_int64, i32, vp]),
        "bci_op_sparse_topk": (st, [vp, vp, ctypes.c_int64, i32, vp, vp]),
        "bci_op_sparse_attention": (st, [vp, vp, i32, vp, i32, vp, vp]),
        "bci_op_transpose_bf16": (st, [vp, vp, vp, i32, i32, i32, vp]),
        "bci_op_add_rmsnorm_backward": (st, [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, ctypes.c_float, vp]),
        "bci_op_silu_mul_backward": (st, [vp, vp, vp, vp, i32, i32, vp]),
        "bci_op_logprob_backward_dz": (st, [vp, vp, vp, vp, i32, i32, vp, vp]),
        "bci_op_rope_backward": (st, [vp, vp, vp, vp, vp, vp]),
        "bci_op_attention_backward": (st, [vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp]),
        "bci_ssd_create": (st, [ctypes.POINTER(SsdConfig), i32, ctypes.POINTER(vp)]),
        "bci_ssd_destroy": (None, [vp]),
        "bci_ssd_last_error": (ctypes.c_char_p, [vp]),
        "bci_ssd_slot_bytes": (ctypes.c_uint64, [vp, i32]),
        "bci_ssd_set_batch": (st, [vp, i32, _P32, _P32, _P32, vp]),
        "bci_ssd_forward": (st, [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp]),
        "bci_profile_begin": (st, [vp, i32]),
        "bci_measure_mfma_rate": (st, [i32, i32, ctypes.POINTER(ctypes.c_double)]),
        "bci_profile_end": (st, [vp, ctypes.POINTER(ctypes.c_double), _P32, ctypes.POINTER(ctypes.c_int64), _P32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


# ------------------------------------------------------------- marshalling

def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        if x.device.type != "cuda":
            raise ValueError("tensor argument must live on the GPU")
        if not x.is_contiguous():
            raise ValueError("tensor argument must be contiguous")
        return x.data_ptr()
    raise TypeError(f"cannot pass {type(x)} as a device pointer")


def _stream(s) -> Optional[int]:
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(ctx, status: int):
    if status != BCI_OK:
        msg = load().bci_last_error(ctx).decode() if ctx else ""
        raise BciError(status, msg)


# ------------------------------------------------------------- entry points

def bci_create(cfg: ModelConfig, device: int = 0) -> int:
    h = ctypes.c_void_p()
    st = load().bci_create(ctypes.byref(cfg), device, ctypes.byref(h))
    if st != BCI_OK:
        raise BciError(st, "bci_create rejected the configuration or could not allocate")
    return h.value


def bci_destroy(ctx: int) -> None:
    load().bci_destroy(ctx)


def bci_last_error(ctx: int) -> str:
    return load().bci_last_error(ctx).decode()


def bci_workspace_bytes(ctx: int) -> int:
    return int(load().bci_workspace_bytes(ctx))


def bci_bind_weights(ctx: int, tensors: Sequence, weight_version: int) -> None:
    arr = (ctypes.c_void_p * len(tensors))(*[_ptr(t) for t in tensors])
    _check(ctx, load().bci_bind_weights(ctx, arr, len(tensors), weight_version))


def bci_weight_version(ctx: int) -> int:
    return int(load().bci_weight_version(ctx))


def bci_bind_kv_cache(ctx: int, k, v, k_scale, v_scale, n_blocks: int) -> None:
    _check(ctx, load().bci_bind_kv_cache(ctx, _ptr(k), _ptr(v), _ptr(k_scale), _ptr(v_scale), n_blocks))


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def bci_set_batch(ctx: int, tokens, cu_q, pos0, block_table, score_rows, score_ids,
                  stream=None) -> None:
    """Host arrays (numpy-like).  block_table is [n_seqs, max_blocks_per_seq]."""
    keep = [_i32(tokens), _i32(cu_q), _i32(pos0), _i32(block_table), _i32(score_rows),
            _i32(score_ids)]
    bt = keep[3].reshape(len(keep[2]), -1) if keep[3].size else keep[3].reshape(len(keep[2]), 0)
    b = Batch()
    b.n_seqs = len(keep[2])
    b.n_tokens = len(keep[0])
    b.n_scored = len(keep[4])
    b.max_blocks_per_seq = bt.shape[1]
    for name, a in zip(("tokens", "cu_q", "pos0", "block_table", "score_rows", "score_ids"), keep):
        setattr(b, name, a.ctypes.data_as(_P32) if a.size else None)
    _check(ctx, load().bci_set_batch(ctx, ctypes.byref(b), _stream(stream)))


def bci_forward_logprobs(ctx: int, logprobs, stream=None) -> None:
    _check(ctx, load().bci_forward_logprobs(ctx, _ptr(logprobs), _stream(stream)))


def bci_forward_logprobs_graph(ctx: int, logprobs, stream=None) -> None:
    _check(ctx, load().bci_forward_logprobs_graph(ctx, _ptr(logprobs), _stream(stream)))


def bci_graph_count(ctx: int) -> int:
    return int(load().bci_graph_count(ctx))


def bci_graph_reset(ctx: int) -> None:
    _check(ctx, load().bci_graph_reset(ctx))


def bci_op_embed(ctx: int, E, r, stream=None) -> None:
    _check(ctx, load().bci_op_embed(ctx, _ptr(E), _ptr(r), _stream(stream)))


def bci_op_add_rmsnorm(ctx: int, a, r, h, g, rows: int, cols: int, eps: float, stream=None) -> None:
    _check(ctx, load().bci_op_add_rmsnorm(ctx, _ptr(a), _ptr(r), _ptr(h), _ptr(g), rows, cols, eps,
                                          _stream(stream)))


def bci_op_gemm_bf16(ctx: int, A, W, C, M: int, N: int, K: int, epilogue: int, stream=None) -> None:
    _check(ctx, load().bci_op_gemm_bf16(ctx, _ptr(A), _ptr(W), _ptr(C), M, N, K, epilogue,
                                        _stream(stream)))


def bci_op_gemm_bf16_ksplit(ctx: int, A, W, C, M: int, N: int, K: int, k_split: int, epilogue: int,
                            workspace, stream=None) -> None:
    _check(ctx, load().bci_op_gemm_bf16_ksplit(ctx, _ptr(A), _ptr(W), _ptr(C), M, N, K, k_split, epilogue,
                                               _ptr(workspace), _stream(stream)))


def bci_op_rope_kv_write(ctx: int, qkv, q_out, layer: int, stream=None) -> None:
    _check(ctx, load().bci_op_rope_kv_write(ctx, _ptr(qkv), _ptr(q_out), layer, _stream(stream)))


def bci_op_kv_gather_dequant(ctx: int, seq: int, n_pos: int, layer: int, k_out, v_out,
                             stream=None) -> None:
    _check(ctx, load().bci_op_kv_gather_dequant(ctx, seq, n_pos, layer, _ptr(k_out), _ptr(v_out),
                                                _stream(stream)))


def bci_op_attention(ctx: int, q, layer: int, o, stream=None) -> None:
    _check(ctx, load().bci_op_attention(ctx, _ptr(q), layer, _ptr(o), _stream(stream)))


def bci_op_gather_scored(ctx: int, src, cols: int, out, stream=None) -> None:
    _check(ctx, load().bci_op_gather_scored(ctx, _ptr(src), cols, _ptr(out), _stream(stream)))


def bci_op_lmhead_logprob(ctx: int, hf, E, ids, M: int, H: int, V: int, lp, stream=None) -> None:
    _check(ctx, load().bci_op_lmhead_logprob(ctx, _ptr(hf), _ptr(E), _ptr(ids), M, H, V, _ptr(lp),
                                             _stream(stream)))


BCI_LMHEAD_NOALLOC_MAX_ROWS, BCI_LMHEAD_NOALLOC_MAX_PAIRS = 1024, 304128


def bci_lmhead_logprob_noalloc(hf, E, ids, M: int, H: int, V: int, lp, stream=None) -> None:
    """No context, no allocation: the partials live in the library's fixed device array."""
    st = load().bci_lmhead_logprob_noalloc(_ptr(hf), _ptr(E), _ptr(ids), M, H, V, _ptr(lp),
                                           _stream(stream))
    if st != BCI_OK:
        raise BciError(st, "bci_lmhead_logprob_noalloc rejected the call (see bci.h for its limits)")


def bci_op_moe_topk(ctx: int, logits, T: int, ids, w, stream=None) -> None:
    _check(ctx, load().bci_op_moe_topk(ctx, _ptr(logits), T, _ptr(ids), _ptr(w), _stream(stream)))


def bci_op_moe_forward(ctx: int, h, ids, w, T: int, wgu, wd, swgu, swd, out, stream=None) -> None:
    _check(ctx, load().bci_op_moe_forward(ctx, _ptr(h), _ptr(ids), _ptr(w), T, _ptr(wgu), _ptr(wd),
                                          _ptr(swgu), _ptr(swd), _ptr(out), _stream(stream)))


def bci_op_index_key_write(ctx: int, kidx, index_dim: int, icodes, iscale, n_index_blocks: int,
                           stream=None) -> None:
    _check(ctx, load().bci_op_index_key_write(ctx, _ptr(kidx), index_dim, _ptr(icodes), _ptr(iscale),
                                              n_index_blocks, _stream(stream)))


def bci_op_index_scores(ctx: int, qidx, w, index_heads: int, index_dim: int, icodes, iscale,
                        n_index_blocks: int, scores, score_stride: int, schedule: int = 0,
                        stream=None) -> None:
    _check(ctx, load().bci_op_index_scores(ctx, _ptr(qidx), _ptr(w), index_heads, index_dim,
                                           _ptr(icodes), _ptr(iscale), n_index_blocks, _ptr(scores),
                                           score_stride, schedule, _stream(stream)))


def bci_op_sparse_topk(ctx: int, scores, score_stride: int, topk: int, sel, stream=None) -> None:
    _check(ctx, load().bci_op_sparse_topk(ctx, _ptr(scores), score_stride, topk, _ptr(sel),
                                          _stream(stream)))


def bci_op_sparse_attention(ctx: int, q, layer: int, sel, topk: int, o, stream=None) -> None:
    _check(ctx, load().bci_op_sparse_attention(ctx, _ptr(q), layer, _ptr(sel), topk, _ptr(o),
                                               _stream(stream)))


def bci_op_transpose_bf16(ctx: int, src, dst, R: int, C: int, ld_dst: int, stream=None) -> None:
    _check(ctx, load().bci_op_transpose_bf16(ctx, _ptr(src), _ptr(dst), R, C, ld_dst, _stream(stream)))


def bci_op_add_rmsnorm_backward(ctx: int, r, g, dh, dr_in, dr, rstd, dg, rows: int, cols: int,
                                eps: float, stream=None) -> None:
    _check(ctx, load().bci_op_add_rmsnorm_backward(ctx, _ptr(r), _ptr(g), _ptr(dh), _ptr(dr_in),
                                                   _ptr(dr), _ptr(rstd), _ptr(dg), rows, cols, eps,
                                                   _stream(stream)))


def bci_op_silu_mul_backward(ctx: int, gu, dact, dgu, rows: int, inter: int, stream=None) -> None:
    _check(ctx, load().bci_op_silu_mul_backward(ctx, _ptr(gu), _ptr(dact), _ptr(dgu), rows, inter,
                                                _stream(stream)))


def bci_op_rope_backward(ctx: int, dq, dk, dv, dqkv, stream=None) -> None:
    _check(ctx, load().bci_op_rope_backward(ctx, _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dqkv), _stream(stream)))


def bci_op_logprob_backward_dz(ctx: int, z, ids, gout, M: int, V: int, dz, stream=None) -> None:
    _check(ctx, load().bci_op_logprob_backward_dz(ctx, _ptr(z), _ptr(ids), _ptr(gout), M, V,
                                                  _ptr(dz), _stream(stream)))


def bci_op_attention_backward(ctx: int, q, k, v, o, dout, L: int, dq, dk, dv, workspace=None,
                              stream=None) -> None:
    _check(ctx, load().bci_op_attention_backward(ctx, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), L,
                                                 _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                                                 _stream(stream)))


def _ssd_check(ctx, status: int):
    if status != BCI_OK:
        msg = load().bci_ssd_last_error(ctx).decode() if ctx else ""
        raise BciError(status, msg)


def bci_ssd_create(cfg: SsdConfig, device: int = 0) -> int:
    h = ctypes.c_void_p()
    st = load().bci_ssd_create(ctypes.byref(cfg), device, ctypes.byref(h))
    if st != BCI_OK:
        raise BciError(st, "bci_ssd_create rejected the configuration or could not allocate")
    return h.value


def bci_ssd_destroy(ctx: int) -> None:
    load().bci_ssd_destroy(ctx)


def bci_ssd_last_error(ctx: int) -> str:
    return load().bci_ssd_last_error(ctx).decode()


def bci_ssd_slot_bytes(ctx: int, which: int) -> int:
    return int(load().bci_ssd_slot_bytes(ctx, which))


def bci_ssd_set_batch(ctx: int, cu_q, pos0, slot, stream=None) -> None:
    """Host arrays: cu_q [n_seqs + 1], pos0 [n_seqs], slot [n_seqs]."""
    keep = [_i32(cu_q), _i32(pos0), _i32(slot)]
    n = len(keep[1])
    _ssd_check(ctx, load().bci_ssd_set_batch(ctx, n, *[a.ctypes.data_as(_P32) for a in keep],
                                             _stream(stream)))


def bci_ssd_forward(ctx: int, x, dt, A, B, C, D, state, chunk_buf, n_slots: int, y,
                    stream=None) -> None:
    _ssd_check(ctx, load().bci_ssd_forward(ctx, _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
                                           _ptr(D), _ptr(state), _ptr(chunk_buf), n_slots, _ptr(y),
                                           _stream(stream)))


def bci_measure_mfma_rate(device: int = 0, random_operands: bool = True) -> float:
    """Sustained dense bf16 MFMA rate of the device in TFLOP/s (see bci.h)."""
    t = ctypes.c_double()
    st = load().bci_measure_mfma_rate(device, int(bool(random_operands)), ctypes.byref(t))
    if st != BCI_OK:
        raise BciError(st, "bci_measure_mfma_rate failed")
    return float(t.value)


def bci_profile_begin(ctx: int, capacity: int = 0) -> None:
    _check(ctx, load().bci_profile_begin(ctx, capacity))


def bci_profile_end(ctx: int):
    """(summed kernel ms, launches timed, sum of their M, launches not timed)."""
    ms = ctypes.c_double()
    n = ctypes.c_int32()
    rows = ctypes.c_int64()
    dropped = ctypes.c_int32()
    _check(ctx, load().bci_profile_end(ctx, ctypes.byref(ms), ctypes.byref(n), ctypes.byref(rows),
                                       ctypes.byref(dropped)))
    return float(ms.value), int(n.value), int(rows.value), int(dropped.value)
