"""Thin Python binding of librq.so (argument marshalling only).

Every function has the name of the C entry point it calls (see include/rq.h) and
takes torch tensors that already live on the GPU; it passes their device pointers
and sizes through ctypes and raises RQError on a non-zero status.  No computation
happens here: if the library is missing the import fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librq.so")

if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is not built; run __graft_entry__.build() or "
                      "python -m looped_transformer_decode_amd.build")
_lib = ctypes.CDLL(_LIB_PATH)

EXPORTS = ("rq_cache_bytes", "rq_workspace_bytes", "rq_bf16_workspace_bytes", "rq_status_str",
           "rq_quantize_token", "rq_decode_attention", "rq_bf16_decode_attention", "rq_unpack_debug",
           "rq_stream_read", "rq_paged_block_bytes", "rq_quantize_token_paged", "rq_decode_attention_paged",
           "rq_kv_project", "rq_decode_attention_noalloc", "rq_w4_weight_bytes", "rq_w4a4_act_bytes",
           "rq_w4a4_workspace_bytes", "rq_w4_quantize_weights", "rq_w4a4_linear")


class rq_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "head_dim", "group", "anchor_bits", "resid_bits", "loops_per_group", "n_groups", "chained",
        "n_kv_heads", "n_q_heads", "max_batch", "max_ctx", "scale_rule")] + [
        ("resid_bits_loop", ctypes.c_int32 * 16)]


class rq_bf16_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("head_dim", "n_kv_heads", "n_q_heads", "max_batch", "t_cap")]


class rq_w4a4_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("in_features", "out_features", "max_tokens")]


class RQError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {rq_status_str(status)} (status {status})")
        self.status = status


_vp, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
_cfgp = ctypes.POINTER(rq_config)
_bcfgp = ctypes.POINTER(rq_bf16_config)

_lib.rq_cache_bytes.argtypes = [_cfgp]
_lib.rq_cache_bytes.restype = _sz
_lib.rq_workspace_bytes.argtypes = [_cfgp]
_lib.rq_workspace_bytes.restype = _sz
_lib.rq_bf16_workspace_bytes.argtypes = [_bcfgp]
_lib.rq_bf16_workspace_bytes.restype = _sz
_lib.rq_status_str.argtypes = [_i32]
_lib.rq_status_str.restype = ctypes.c_char_p
_lib.rq_quantize_token.argtypes = [_cfgp, _vp, _vp, ctypes.POINTER(ctypes.c_int64), _i32, _vp, _vp,
                                   _i32, _i32, _vp]
_lib.rq_quantize_token.restype = _i32
_lib.rq_decode_attention.argtypes = [_cfgp, _vp, _i32, _vp, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _f32,
                                     _vp, _vp, _sz, _i32, _i32, _vp]
_lib.rq_decode_attention.restype = _i32
_lib.rq_decode_attention_noalloc.argtypes = [_cfgp, _vp, _i32, _vp, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _f32, _vp,
                                             _i32, _i32, _vp]
_lib.rq_decode_attention_noalloc.restype = _i32
_lib.rq_bf16_decode_attention.argtypes = [_bcfgp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _vp, _i32, _f32,
                                          _vp, _vp, _sz, _i32, _i32, _vp]
_lib.rq_bf16_decode_attention.restype = _i32
_lib.rq_unpack_debug.argtypes = [_cfgp, _vp, _i32, _vp, _i32, _i32, _i32, _vp, _vp]
_lib.rq_unpack_debug.restype = _i32
_lib.rq_stream_read.argtypes = [_vp, _sz, _vp, _sz, _vp]
_lib.rq_stream_read.restype = _i32
_lib.rq_paged_block_bytes.argtypes = [_cfgp]
_lib.rq_paged_block_bytes.restype = _sz
_lib.rq_quantize_token_paged.argtypes = [_cfgp, _vp, _i32, _vp, _i32, _vp, ctypes.POINTER(ctypes.c_int64), _i32, _vp,
                                         _vp, _i32, _i32, _vp]
_lib.rq_quantize_token_paged.restype = _i32
_lib.rq_decode_attention_paged.argtypes = [_cfgp, _vp, _i32, _vp, _i32, _i32, _vp, _i32, _vp, _vp, _vp, _vp, _i32,
                                           _vp, _f32, _vp, _vp, _sz, _i32, _i32, _vp]
_lib.rq_decode_attention_paged.restype = _i32
_lib.rq_kv_project.argtypes = [_cfgp, _vp, ctypes.c_int64, _i32, _vp, _i32, _vp, _vp, _vp, _i32, _vp]
_lib.rq_kv_project.restype = _i32
_wcfgp = ctypes.POINTER(rq_w4a4_config)
for _fn in ("rq_w4_weight_bytes", "rq_w4a4_act_bytes", "rq_w4a4_workspace_bytes"):
    getattr(_lib, _fn).argtypes = [_wcfgp]
    getattr(_lib, _fn).restype = _sz
_lib.rq_w4_quantize_weights.argtypes = [_wcfgp, _vp, ctypes.c_int64, _vp, _vp, _vp]
_lib.rq_w4_quantize_weights.restype = _i32
_lib.rq_w4a4_linear.argtypes = [_wcfgp, _vp, _vp, ctypes.c_int64, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp,
                                _sz, _vp]
_lib.rq_w4a4_linear.restype = _i32


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise RQError(fn, status)


def rq_status_str(status: int) -> str:
    return _lib.rq_status_str(int(status)).decode()


def rq_cache_bytes(cfg: rq_config) -> int:
    return int(_lib.rq_cache_bytes(ctypes.byref(cfg)))


def rq_workspace_bytes(cfg: rq_config) -> int:
    return int(_lib.rq_workspace_bytes(ctypes.byref(cfg)))


def rq_bf16_workspace_bytes(cfg: rq_bf16_config) -> int:
    return int(_lib.rq_bf16_workspace_bytes(ctypes.byref(cfg)))


def rq_quantize_token(cfg: rq_config, cache: torch.Tensor, pending: torch.Tensor, group_idx: int,
                      pos: torch.Tensor, rot: torch.Tensor, batch: int, n_tokens: int = 1,
                      pending_strides: Optional[Sequence[int]] = None, stream=None) -> None:
    st = None
    if pending_strides is not None:
        st = (ctypes.c_int64 * 5)(*[int(s) for s in pending_strides])
    _check("rq_quantize_token", _lib.rq_quantize_token(
        ctypes.byref(cfg), _ptr(cache), _ptr(pending), st, group_idx, _ptr(pos), _ptr(rot),
        batch, n_tokens, _stream(stream)))


def rq_decode_attention(cfg: rq_config, cache: torch.Tensor, loop: int, q: torch.Tensor,
                        k_cur: torch.Tensor, v_cur: torch.Tensor, pending: Optional[torch.Tensor],
                        ctx_len: torch.Tensor, ctx_bound: int, rot: torch.Tensor, sm_scale: float,
                        out: torch.Tensor, workspace: torch.Tensor, batch: int, n_splits: int = 0,
                        stream=None) -> None:
    q_bf16 = 1 if q.dtype == torch.bfloat16 else 0
    _check("rq_decode_attention", _lib.rq_decode_attention(
        ctypes.byref(cfg), _ptr(cache), loop, _ptr(q), q_bf16, _ptr(k_cur), _ptr(v_cur), _ptr(pending),
        _ptr(ctx_len), ctx_bound, _ptr(rot), sm_scale, _ptr(out), _ptr(workspace), _nbytes(workspace),
        batch, n_splits, _stream(stream)))


def rq_decode_attention_noalloc(cfg: rq_config, cache: torch.Tensor, loop: int, q: torch.Tensor,
                                k_cur: torch.Tensor, v_cur: torch.Tensor, pending: Optional[torch.Tensor],
                                ctx_len: torch.Tensor, ctx_bound: int, rot: torch.Tensor, sm_scale: float,
                                out: torch.Tensor, batch: int, n_splits: int = 0, stream=None) -> None:
    q_bf16 = 1 if q.dtype == torch.bfloat16 else 0
    _check("rq_decode_attention_noalloc", _lib.rq_decode_attention_noalloc(
        ctypes.byref(cfg), _ptr(cache), loop, _ptr(q), q_bf16, _ptr(k_cur), _ptr(v_cur), _ptr(pending),
        _ptr(ctx_len), ctx_bound, _ptr(rot), sm_scale, _ptr(out), batch, n_splits, _stream(stream)))


def rq_bf16_decode_attention(cfg: rq_bf16_config, k_cache: torch.Tensor, v_cache: torch.Tensor,
                             q: torch.Tensor, k_cur: torch.Tensor, v_cur: torch.Tensor, append: bool,
                             ctx_len: torch.Tensor, ctx_bound: int, sm_scale: float, out: torch.Tensor,
                             workspace: torch.Tensor, batch: int, n_splits: int = 0, stream=None) -> None:
    q_bf16 = 1 if q.dtype == torch.bfloat16 else 0
    _check("rq_bf16_decode_attention", _lib.rq_bf16_decode_attention(
        ctypes.byref(cfg), _ptr(k_cache), _ptr(v_cache), _ptr(q), q_bf16, _ptr(k_cur), _ptr(v_cur),
        1 if append else 0, _ptr(ctx_len), ctx_bound, sm_scale, _ptr(out), _ptr(workspace),
        _nbytes(workspace), batch, n_splits, _stream(stream)))


def rq_unpack_debug(cfg: rq_config, cache: torch.Tensor, loop: int, rot: torch.Tensor, t0: int, t1: int,
                    batch: int, out: torch.Tensor, stream=None) -> None:
    _check("rq_unpack_debug", _lib.rq_unpack_debug(
        ctypes.byref(cfg), _ptr(cache), loop, _ptr(rot), t0, t1, batch, _ptr(out), _stream(stream)))


def rq_paged_block_bytes(cfg: rq_config) -> int:
    return int(_lib.rq_paged_block_bytes(ctypes.byref(cfg)))


def rq_quantize_token_paged(cfg: rq_config, pool: torch.Tensor, n_blocks: int, block_table: torch.Tensor,
                            pending: torch.Tensor, group_idx: int, pos: torch.Tensor, rot: torch.Tensor, batch: int,
                            n_tokens: int = 1, pending_strides: Optional[Sequence[int]] = None, stream=None) -> None:
    st = None
    if pending_strides is not None:
        st = (ctypes.c_int64 * 5)(*[int(s) for s in pending_strides])
    _check("rq_quantize_token_paged", _lib.rq_quantize_token_paged(
        ctypes.byref(cfg), _ptr(pool), n_blocks, _ptr(block_table), block_table.shape[1], _ptr(pending), st,
        group_idx, _ptr(pos), _ptr(rot), batch, n_tokens, _stream(stream)))


def rq_decode_attention_paged(cfg: rq_config, pool: torch.Tensor, n_blocks: int, block_table: torch.Tensor,
                              loop: int, q: torch.Tensor, k_cur: torch.Tensor, v_cur: torch.Tensor,
                              pending: Optional[torch.Tensor], ctx_len: torch.Tensor, ctx_bound: int,
                              rot: torch.Tensor, sm_scale: float, out: torch.Tensor, workspace: torch.Tensor,
                              batch: int, n_splits: int = 0, stream=None) -> None:
    q_bf16 = 1 if q.dtype == torch.bfloat16 else 0
    _check("rq_decode_attention_paged", _lib.rq_decode_attention_paged(
        ctypes.byref(cfg), _ptr(pool), n_blocks, _ptr(block_table), block_table.shape[1], loop, _ptr(q), q_bf16,
        _ptr(k_cur), _ptr(v_cur), _ptr(pending), _ptr(ctx_len), ctx_bound, _ptr(rot), sm_scale, _ptr(out),
        _ptr(workspace), _nbytes(workspace), batch, n_splits, _stream(stream)))


def rq_kv_project(cfg: rq_config, x: torch.Tensor, w_kv: torch.Tensor, loop: int,
                  k_cur: Optional[torch.Tensor], v_cur: Optional[torch.Tensor], pending: Optional[torch.Tensor],
                  batch: int, stream=None) -> None:
    """x: [batch][hidden] BF16 (any row stride); w_kv: [2][Hkv][d][hidden] BF16; k_cur, v_cur:
    [batch][Hkv][d] BF16; pending: [>= batch][L][2][Hkv][d] BF16 (the library writes through
    these pointers, so their shapes are checked here)."""
    if x.dtype != torch.bfloat16 or w_kv.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("rq_kv_project: x must be a BF16 [batch][hidden] tensor with unit channel stride")
    hidden = x.shape[1]
    hkv, d, L = cfg.n_kv_heads, cfg.head_dim, cfg.loops_per_group
    if not w_kv.is_contiguous() or tuple(w_kv.shape) != (2, hkv, d, hidden):
        raise ValueError("rq_kv_project: w_kv must be a contiguous [2][Hkv][d][hidden] BF16 tensor")
    if x.shape[0] < batch:
        raise ValueError("rq_kv_project: x has fewer rows than batch")
    for name, t, shape in (("k_cur", k_cur, (batch, hkv, d)), ("v_cur", v_cur, (batch, hkv, d))):
        if t is not None and (t.dtype != torch.bfloat16 or not t.is_contiguous() or t.numel() < batch * hkv * d
                              or tuple(t.shape[1:]) != shape[1:] or t.device != x.device):
            raise ValueError(f"rq_kv_project: {name} must be a contiguous BF16 [batch][Hkv][d] tensor on x's device")
    if pending is not None and (pending.dtype != torch.bfloat16 or not pending.is_contiguous()
                                or tuple(pending.shape[1:]) != (L, 2, hkv, d) or pending.shape[0] < batch
                                or pending.device != x.device):
        raise ValueError("rq_kv_project: pending must be a contiguous BF16 [batch][L][2][Hkv][d] tensor on x's device")
    if w_kv.device != x.device:
        raise ValueError("rq_kv_project: x and w_kv must be on the same device")
    _check("rq_kv_project", _lib.rq_kv_project(
        ctypes.byref(cfg), _ptr(x), x.stride(0), hidden, _ptr(w_kv), loop, _ptr(k_cur), _ptr(v_cur), _ptr(pending),
        batch, _stream(stream)))


STREAM_SINK_WORDS = 1 << 20


def rq_stream_read(buf: torch.Tensor, nbytes: int, sink: torch.Tensor, stream=None) -> None:
    _check("rq_stream_read", _lib.rq_stream_read(_ptr(buf), nbytes, _ptr(sink), sink.numel(), _stream(stream)))


def config_for(wl, chained: Optional[bool] = None, max_batch: Optional[int] = None,
               max_ctx: Optional[int] = None) -> rq_config:
    """rq_config for a synth.Workload (capacity: its batch, context + the current token)."""
    widths = tuple(getattr(wl, "resid_bits_loop", ()) or ())
    return rq_config(wl.head_dim, wl.group, wl.anchor_bits, wl.resid_bits, wl.loops_per_group,
                     wl.n_groups, int(wl.chained if chained is None else chained), wl.n_kv_heads,
                     wl.n_q_heads, max_batch or wl.batch, max_ctx or wl.ctx + 1, wl.scale_rule,
                     (ctypes.c_int32 * 16)(*widths))


def bf16_config_for(wl, max_batch: Optional[int] = None, t_cap: Optional[int] = None) -> rq_bf16_config:
    return rq_bf16_config(wl.head_dim, wl.n_kv_heads, wl.n_q_heads, max_batch or wl.batch,
                          t_cap or wl.ctx + 1)


# ---- W4A4 linear layer with cross-loop residual activations

def w4a4_config(in_features: int, out_features: int, max_tokens: int) -> rq_w4a4_config:
    return rq_w4a4_config(in_features, out_features, max_tokens)


def rq_w4_weight_bytes(cfg: rq_w4a4_config) -> int:
    return int(_lib.rq_w4_weight_bytes(ctypes.byref(cfg)))


def rq_w4a4_act_bytes(cfg: rq_w4a4_config) -> int:
    return int(_lib.rq_w4a4_act_bytes(ctypes.byref(cfg)))


def rq_w4a4_workspace_bytes(cfg: rq_w4a4_config) -> int:
    return int(_lib.rq_w4a4_workspace_bytes(ctypes.byref(cfg)))


def _need(name: str, t: Optional[torch.Tensor], dtype, numel: int, dev) -> None:
    if t is None:
        return
    if t.dtype != dtype or not t.is_contiguous() or t.numel() < numel or t.device != dev:
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of >= {numel} elements on {dev}")


def rq_w4_quantize_weights(cfg: rq_w4a4_config, w: torch.Tensor, rot: Optional[torch.Tensor], out: torch.Tensor,
                           stream=None) -> None:
    """w: BF16 [out_features][>= in_features] (unit channel stride); rot: float32 [128][128] or None;
    out: uint8 of rq_w4_weight_bytes(cfg) bytes."""
    if w.dtype != torch.bfloat16 or w.dim() != 2 or w.stride(1) != 1 or w.shape[0] != cfg.out_features \
            or w.shape[1] < cfg.in_features:
        raise ValueError("rq_w4_quantize_weights: w must be a BF16 [out_features][in_features] tensor")
    _need("rq_w4_quantize_weights: out", out, torch.uint8, rq_w4_weight_bytes(cfg), w.device)
    _need("rq_w4_quantize_weights: rot", rot, torch.float32, 128 * 128, w.device)
    _check("rq_w4_quantize_weights", _lib.rq_w4_quantize_weights(
        ctypes.byref(cfg), _ptr(w), w.stride(0), _ptr(rot), _ptr(out), _stream(stream)))


def rq_w4a4_linear(cfg: rq_w4a4_config, weights: torch.Tensor, x: torch.Tensor, loop_local: int,
                   anchor: torch.Tensor, act: Optional[torch.Tensor], rot: Optional[torch.Tensor],
                   c_out: Optional[torch.Tensor], y0: torch.Tensor, y: torch.Tensor, n_tokens: int,
                   workspace: torch.Tensor, stream=None) -> None:
    """x: BF16 [>= n_tokens][>= in_features] (unit channel stride); anchor, act: uint8 activation
    rows; y0, y: float32 [n_tokens][out_features]; c_out: float32 [n_tokens] or None."""
    dev = x.device
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1 or x.shape[0] < n_tokens \
            or x.shape[1] < cfg.in_features:
        raise ValueError("rq_w4a4_linear: x must be a BF16 [tokens][in_features] tensor")
    _need("rq_w4a4_linear: weights", weights, torch.uint8, rq_w4_weight_bytes(cfg), dev)
    _need("rq_w4a4_linear: anchor", anchor, torch.uint8, rq_w4a4_act_bytes(cfg), dev)
    _need("rq_w4a4_linear: act", act, torch.uint8, rq_w4a4_act_bytes(cfg), dev)
    _need("rq_w4a4_linear: rot", rot, torch.float32, 128 * 128, dev)
    _need("rq_w4a4_linear: c_out", c_out, torch.float32, n_tokens, dev)
    _need("rq_w4a4_linear: y0", y0, torch.float32, n_tokens * cfg.out_features, dev)
    _need("rq_w4a4_linear: y", y, torch.float32, n_tokens * cfg.out_features, dev)
    _need("rq_w4a4_linear: workspace", workspace, torch.uint8, 1, dev)
    _check("rq_w4a4_linear", _lib.rq_w4a4_linear(
        ctypes.byref(cfg), _ptr(weights), _ptr(x), x.stride(0), loop_local, _ptr(anchor), _ptr(act), _ptr(rot),
        _ptr(c_out), _ptr(y0), _ptr(y), n_tokens, _ptr(workspace), _nbytes(workspace), _stream(stream)))
