"""Python binding of the MI355X bifocal-attention library (``libjetlong.so``).

Argument marshalling only: every function here takes torch tensors that the
caller has allocated on the GPU, passes their device pointers, sizes and the
current HIP stream to the C ABI of the same name (``include/jl_bifocal.h``),
and raises :class:`JetLongError` on a non-zero status.  All computation runs in
the library's HIP kernels; there is no fallback.  The library is loaded on
first use and must have been built (``zero_shot_rope_attention_amd.build``).
"""

from __future__ import annotations

import ctypes
import os

__all__ = [
    "JetLongError",
    "LIB_PATH",
    "EXPORTED_SYMBOLS",
    "load_library",
    "jl_group_factor",
    "jl_bifocal_prefill",
    "jl_bifocal_prefill_workspace_size",
    "jl_bifocal_prefill_ws",
    "jl_plain_prefill",
    "jl_bifocal_prefill_passes",
    "jl_bifocal_prefill_three_pass",
    "jl_bifocal_decode_workspace_size",
    "jl_bifocal_decode",
    "jl_plain_decode",
    "jl_bifocal_decode_noalloc",
    "jl_bifocal_decode_varlen",
    "jl_plain_decode_varlen",
    "jl_sliding_prefill",
    "jl_sliding_decode",
    "SCHEDULES",
    "jl_schedule_factor",
    "jl_bifocal_prefill_sched",
    "jl_bifocal_decode_sched",
    "jl_bifocal_prefill_varlen",
    "jl_plain_prefill_varlen",
    "jl_bifocal_prefill_positions",
    "jl_plain_prefill_positions",
    "jl_bifocal_decode_paged",
    "jl_plain_decode_paged",
    "jl_qwen3_layer_workspace_size",
    "jl_qwen3_attention_layer",
]

# JL_LIBRARY may name another build of the same library (the host-sanitized one)
LIB_PATH = os.environ.get("JL_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libjetlong.so")

_i32, _i64, _f32, _f64, _vp, _sz = (ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double,
                                    ctypes.c_void_p, ctypes.c_size_t)

# name -> (restype, argtypes); must match include/jl_bifocal.h
_SIGNATURES = {
    "jl_last_error": (ctypes.c_char_p, []),
    "jl_group_factor": (_i64, [_i64, _i64]),
    "jl_bifocal_prefill": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i64, _i64,
                                  _f64, _f32, _vp]),
    "jl_bifocal_prefill_workspace_size": (_sz, [_i32, _i32, _i32, _i32]),
    "jl_bifocal_prefill_ws": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i64, _i64, _f64,
                                     _f32, _vp, _sz, _vp]),
    "jl_plain_prefill": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _vp]),
    "jl_bifocal_prefill_passes": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i64, _i64,
                                         _f64, _f32, _vp]),
    "jl_bifocal_prefill_three_pass": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i64,
                                             _i64, _f64, _f32, _vp]),
    "jl_bifocal_decode_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "jl_bifocal_decode": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i64, _i64, _f64, _f32,
                                 _vp, _sz, _vp]),
    "jl_plain_decode": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _f32, _vp, _sz, _vp]),
    "jl_bifocal_decode_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i64, _i64, _f64,
                                         _f32, _vp]),
    "jl_bifocal_decode_varlen": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i64, _i64, _f64,
                                        _f32, _vp, _sz, _vp]),
    "jl_plain_decode_varlen": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _f32, _vp, _sz,
                                      _vp]),
    "jl_sliding_prefill": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i64, _f32, _vp]),
    "jl_sliding_decode": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i64, _f32, _vp, _sz, _vp]),
    "jl_schedule_factor": (ctypes.c_double, [_i64, _i64, _i64, _i32]),
    "jl_bifocal_prefill_sched": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i64, _i64,
                                        _f64, _i32, _f32, _vp, _sz, _vp]),
    "jl_bifocal_decode_sched": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i64, _i64,
                                       _f64, _i32, _f32, _vp, _sz, _vp]),
    "jl_bifocal_prefill_varlen": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                         _i32, _i64, _i64, _f64, _i32, _f32, _vp, _sz, _vp]),
    "jl_plain_prefill_varlen": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                       _f32, _vp]),
    "jl_bifocal_prefill_positions": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i64,
                                            _i64, _f64, _i32, _f32, _vp, _sz, _vp]),
    "jl_plain_prefill_positions": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                                          _vp]),
    "jl_bifocal_decode_paged": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                       _i64, _i64, _f64, _i32, _f32, _vp, _sz, _vp]),
    "jl_plain_decode_paged": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                     _f32, _vp, _sz, _vp]),
    "jl_qwen3_layer_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "jl_qwen3_attention_layer": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                        _i32, _f32, _i32, _i64, _i64, _f64, _i32, _vp, _sz, _vp]),
}
EXPORTED_SYMBOLS = tuple(_SIGNATURES)

_STATUS = {1: "JL_ERR_INVALID_ARG", 2: "JL_ERR_UNSUPPORTED", 3: "JL_ERR_WORKSPACE", 4: "JL_ERR_DEVICE"}
_lib = None


class JetLongError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libjetlong.so (once) and declare its C signatures.  Raises if it has
    not been built: there is no fallback implementation."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with `python -m zero_shot_rope_attention_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(status: int) -> None:
    if status != 0:
        msg = load_library().jl_last_error()
        raise JetLongError(status, msg.decode() if msg else "")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous device tensors")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def jl_group_factor(seq_len: int, pretrained_window: int) -> int:
    return int(load_library().jl_group_factor(int(seq_len), int(pretrained_window)))


def jl_bifocal_prefill(q, k, v, out, lse, pretrained_window, local_window, rope_base,
                       softmax_scale=0.0, stream=None, q_pos=None):
    """q [B, n_q, Hq, D], k/v [B, n_kv, Hkv, D] bf16; out like q; lse fp32 [B, Hq, n_q] or None;
    q_pos None (the newest n_q positions) or an int32 device tensor [n_q] of query positions."""
    b, n_q, hq, d = q.shape
    n_kv, hkv = k.shape[1], k.shape[2]
    _check(load_library().jl_bifocal_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _pos_ptr(q_pos), b,
                                             n_q, n_kv, hq, hkv, d, int(pretrained_window), int(local_window),
                                             float(rope_base), float(softmax_scale), _stream(stream)))


def jl_bifocal_prefill_workspace_size(batch, n_kv, n_kv_heads, head_dim=128) -> int:
    return int(load_library().jl_bifocal_prefill_workspace_size(batch, n_kv, n_kv_heads, head_dim))


def jl_bifocal_prefill_ws(q, k, v, out, lse, pretrained_window, local_window, rope_base, workspace,
                          softmax_scale=0.0, stream=None):
    """As jl_bifocal_prefill, with the corrected keys written to `workspace` (a device
    tensor of at least jl_bifocal_prefill_workspace_size bytes) by a pass of their own."""
    b, n_q, hq, d = q.shape
    n_kv, hkv = k.shape[1], k.shape[2]
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().jl_bifocal_prefill_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), b, n_q, n_kv, hq,
                                                hkv, d, int(pretrained_window), int(local_window), float(rope_base),
                                                float(softmax_scale), _ptr(workspace), nbytes, _stream(stream)))


def jl_plain_prefill(q, k, v, out, lse, softmax_scale=0.0, stream=None, q_pos=None):
    b, n_q, hq, d = q.shape
    n_kv, hkv = k.shape[1], k.shape[2]
    _check(load_library().jl_plain_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _pos_ptr(q_pos), b, n_q,
                                           n_kv, hq, hkv, d, float(softmax_scale), _stream(stream)))


def jl_bifocal_prefill_passes(q, k, v, out_abc, lse_abc, pretrained_window, local_window, rope_base,
                              softmax_scale=0.0, stream=None):
    """out_abc fp32 [3, B, n_q, Hq, D]; lse_abc fp32 [3, B, Hq, n_q]."""
    b, n_q, hq, d = q.shape
    n_kv, hkv = k.shape[1], k.shape[2]
    _check(load_library().jl_bifocal_prefill_passes(_ptr(q), _ptr(k), _ptr(v), _ptr(out_abc), _ptr(lse_abc), b, n_q,
                                                    n_kv, hq, hkv, d, int(pretrained_window), int(local_window),
                                                    float(rope_base), float(softmax_scale), _stream(stream)))


def jl_bifocal_prefill_three_pass(q, k, v, out, lse, pretrained_window, local_window, rope_base, softmax_scale=0.0,
                                  stream=None):
    """The three passes merged by their lse weights in one kernel: out bf16 [B, n_q, Hq, D]; lse fp32 [B, Hq, n_q]
    or None."""
    b, n_q, hq, d = q.shape
    n_kv, hkv = k.shape[1], k.shape[2]
    _check(load_library().jl_bifocal_prefill_three_pass(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), b, n_q,
                                                        n_kv, hq, hkv, d, int(pretrained_window), int(local_window),
                                                        float(rope_base), float(softmax_scale), _stream(stream)))


def jl_bifocal_decode_workspace_size(batch, n_kv, n_q_heads, n_kv_heads, head_dim=128) -> int:
    return int(load_library().jl_bifocal_decode_workspace_size(batch, n_kv, n_q_heads, n_kv_heads, head_dim))


def jl_bifocal_decode(q, k_cache, v_cache, out, lse, pretrained_window, local_window, rope_base, workspace,
                      softmax_scale=0.0, stream=None):
    """q [B, 1, Hq, D]; caches [B, n_kv, Hkv, D]; workspace: a device tensor of
    at least jl_bifocal_decode_workspace_size bytes."""
    b, _, hq, d = q.shape
    n_kv, hkv = k_cache.shape[1], k_cache.shape[2]
    nbytes = workspace.numel() * workspace.element_size()
    _check(load_library().jl_bifocal_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse), b, n_kv,
                                            hq, hkv, d, int(pretrained_window), int(local_window), float(rope_base),
                                            float(softmax_scale), _ptr(workspace), nbytes, _stream(stream)))


def jl_plain_decode(q, k_cache, v_cache, out, lse, workspace, softmax_scale=0.0, stream=None):
    b, _, hq, d = q.shape
    n_kv, hkv = k_cache.shape[1], k_cache.shape[2]
    nbytes = workspace.numel() * workspace.element_size()
    _check(load_library().jl_plain_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse), b, n_kv, hq,
                                          hkv, d, float(softmax_scale), _ptr(workspace), nbytes, _stream(stream)))


def jl_bifocal_decode_noalloc(q, k_cache, v_cache, out, lse, pretrained_window, local_window, rope_base,
                              softmax_scale=0.0, stream=None):
    """As jl_bifocal_decode, with the library's own device array as the workspace."""
    b, _, hq, d = q.shape
    n_kv, hkv = k_cache.shape[1], k_cache.shape[2]
    _check(load_library().jl_bifocal_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse), b,
                                                    n_kv, hq, hkv, d, int(pretrained_window), int(local_window),
                                                    float(rope_base), float(softmax_scale), _stream(stream)))


def _seq_lens_ptr(seq_lens):
    import torch
    if seq_lens is None:
        return None
    if seq_lens.dtype != torch.int32:
        raise TypeError("seq_lens must be an int32 device tensor")
    return _ptr(seq_lens)


def jl_bifocal_decode_varlen(q, k_cache, v_cache, out, lse, seq_lens, pretrained_window, local_window, rope_base,
                             workspace, softmax_scale=0.0, stream=None):
    """q [B, 1, Hq, D]; caches [B, max_seq_len, Hkv, D]; seq_lens int32 [B] on the
    device (keys held by each sequence); workspace as for jl_bifocal_decode with
    n_kv = max_seq_len."""
    b, _, hq, d = q.shape
    n_max, hkv = k_cache.shape[1], k_cache.shape[2]
    nbytes = workspace.numel() * workspace.element_size()
    _check(load_library().jl_bifocal_decode_varlen(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse), _seq_lens_ptr(seq_lens), b, n_max, hq, hkv, d,
        int(pretrained_window), int(local_window), float(rope_base), float(softmax_scale), _ptr(workspace), nbytes,
        _stream(stream)))


def jl_plain_decode_varlen(q, k_cache, v_cache, out, lse, seq_lens, workspace, softmax_scale=0.0, stream=None):
    b, _, hq, d = q.shape
    n_max, hkv = k_cache.shape[1], k_cache.shape[2]
    nbytes = workspace.numel() * workspace.element_size()
    _check(load_library().jl_plain_decode_varlen(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse), _seq_lens_ptr(seq_lens), b, n_max, hq, hkv, d,
        float(softmax_scale), _ptr(workspace), nbytes, _stream(stream)))


def jl_sliding_prefill(q, k, v, out, lse, local_window, softmax_scale=0.0, stream=None):
    """Sliding-window attention over the newest ``local_window`` keys of each
    query row; layouts as jl_bifocal_prefill."""
    b, n_q, hq, d = q.shape
    n_kv, hkv = k.shape[1], k.shape[2]
    _check(load_library().jl_sliding_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), b, n_q, n_kv, hq, hkv,
                                             d, int(local_window), float(softmax_scale), _stream(stream)))


def jl_sliding_decode(q, k_cache, v_cache, out, lse, local_window, workspace, softmax_scale=0.0, stream=None):
    """One new token over the newest ``local_window`` cached keys; workspace as
    for jl_bifocal_decode."""
    b, _, hq, d = q.shape
    n_kv, hkv = k_cache.shape[1], k_cache.shape[2]
    nbytes = workspace.numel() * workspace.element_size()
    _check(load_library().jl_sliding_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse), b, n_kv, hq,
                                            hkv, d, int(local_window), float(softmax_scale), _ptr(workspace), nbytes,
                                            _stream(stream)))


# Long-range schedules, numbered as in the C header (JL_SCHED_*).
SCHEDULES = {"grouped": 0, "seam": 1, "fractional": 2}


def _schedule_id(schedule) -> int:
    if isinstance(schedule, str):
        if schedule not in SCHEDULES:
            raise ValueError(f"unknown schedule {schedule!r}")
        return SCHEDULES[schedule]
    return int(schedule)


def jl_schedule_factor(seq_len, pretrained_window, local_window, schedule="grouped") -> float:
    """g (integer schedules) or l (fractional) for a sequence of seq_len keys; 0.0 if invalid."""
    return float(load_library().jl_schedule_factor(int(seq_len), int(pretrained_window), int(local_window),
                                                   _schedule_id(schedule)))


def jl_bifocal_prefill_sched(q, k, v, out, lse, pretrained_window, local_window, rope_base, schedule,
                             workspace=None, softmax_scale=0.0, stream=None):
    """Bifocal prefill under a long-range schedule ("grouped", "seam", "fractional");
    with a workspace the two-launch form, without one the single kernel."""
    b, n_q, hq, d = q.shape
    n_kv, hkv = k.shape[1], k.shape[2]
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().jl_bifocal_prefill_sched(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), b, n_q, n_kv, hq, hkv, d, int(pretrained_window),
        int(local_window), float(rope_base), _schedule_id(schedule), float(softmax_scale), _ptr(workspace), nbytes,
        _stream(stream)))


def jl_bifocal_decode_sched(q, k_cache, v_cache, out, lse, seq_lens, pretrained_window, local_window, rope_base,
                            schedule, workspace, softmax_scale=0.0, stream=None):
    """Bifocal decode under a long-range schedule; seq_lens None (every sequence
    holds the whole cache) or an int32 device tensor [B]."""
    b, _, hq, d = q.shape
    n_kv, hkv = k_cache.shape[1], k_cache.shape[2]
    nbytes = workspace.numel() * workspace.element_size()
    _check(load_library().jl_bifocal_decode_sched(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse), _seq_lens_ptr(seq_lens), b, n_kv, hq, hkv, d,
        int(pretrained_window), int(local_window), float(rope_base), _schedule_id(schedule), float(softmax_scale),
        _ptr(workspace), nbytes, _stream(stream)))


def jl_qwen3_layer_workspace_size(batch, n_new, n_kv, n_q_heads, n_kv_heads, head_dim=128) -> int:
    return int(load_library().jl_qwen3_layer_workspace_size(batch, n_new, n_kv, n_q_heads, n_kv_heads, head_dim))


def jl_qwen3_attention_layer(x, w_qkv, q_norm_weight, k_norm_weight, w_o, out, k_cache, v_cache, workspace,
                             bifocal=True, pretrained_window=1, local_window=1, rope_base=1e6, schedule="grouped",
                             rms_eps=1e-6, stream=None):
    """One Qwen3-shaped attention layer over x [B, n_new, hidden], appending to the
    caches [B, n_kv, Hkv, 128] at rows n_kv - n_new ..; out [B, n_new, hidden]."""
    b, n_new, hidden = x.shape
    n_kv, hkv, d = k_cache.shape[1], k_cache.shape[2], k_cache.shape[3]
    hq = w_o.shape[1] // d
    nbytes = workspace.numel() * workspace.element_size()
    _check(load_library().jl_qwen3_attention_layer(
        _ptr(x), _ptr(w_qkv), _ptr(q_norm_weight), _ptr(k_norm_weight), _ptr(w_o), _ptr(out), _ptr(k_cache),
        _ptr(v_cache), b, n_new, n_kv, hidden, hq, hkv, d, float(rms_eps), 1 if bifocal else 0,
        int(pretrained_window), int(local_window), float(rope_base), _schedule_id(schedule), _ptr(workspace), nbytes,
        _stream(stream)))


def _cu_ptr(cu):
    import torch
    if cu.dtype != torch.int32:
        raise TypeError("cu_seqlens_q must be an int32 device tensor")
    return _ptr(cu)


def jl_bifocal_prefill_varlen(q, k_cache, v_cache, out, lse, cu_seqlens_q, seq_lens, max_q, pretrained_window,
                              local_window, rope_base, workspace, schedule="grouped", softmax_scale=0.0, stream=None):
    """q, out [total_q, Hq, D] packed rows; caches [B, max_seq_len, Hkv, D]; lse
    [Hq, total_q] or None; cu_seqlens_q int32 [B+1] and seq_lens int32 [B] on the
    device; max_q >= every sequence's new rows; workspace None (the single-kernel form)
    or as for jl_bifocal_prefill_ws with n_kv = max_seq_len (the two-launch form)."""
    total_q, hq, d = q.shape
    b, n_max, hkv = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().jl_bifocal_prefill_varlen(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse), _cu_ptr(cu_seqlens_q), _seq_lens_ptr(seq_lens), b,
        total_q, int(max_q), n_max, hq, hkv, d, int(pretrained_window), int(local_window), float(rope_base),
        _schedule_id(schedule), float(softmax_scale), _ptr(workspace), nbytes, _stream(stream)))


def jl_plain_prefill_varlen(q, k_cache, v_cache, out, lse, cu_seqlens_q, seq_lens, max_q, softmax_scale=0.0,
                            stream=None):
    total_q, hq, d = q.shape
    b, n_max, hkv = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    _check(load_library().jl_plain_prefill_varlen(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse), _cu_ptr(cu_seqlens_q), _seq_lens_ptr(seq_lens), b,
        total_q, int(max_q), n_max, hq, hkv, d, float(softmax_scale), _stream(stream)))


def _pos_ptr(q_pos):
    if q_pos is None:
        return None
    import torch
    if q_pos.dtype != torch.int32:
        raise TypeError("q_pos must be an int32 device tensor")
    return _ptr(q_pos)


def jl_bifocal_prefill_positions(q, k, v, out, lse, q_pos, pretrained_window, local_window, rope_base,
                                 workspace=None, schedule="grouped", softmax_scale=0.0, stream=None):
    """Query row i at position q_pos[i] (int32 device tensor [n_q], nondecreasing), under
    `schedule`; with a workspace the two-launch form, with workspace None the single kernel."""
    b, n_q, hq, d = q.shape
    n_kv, hkv = k.shape[1], k.shape[2]
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().jl_bifocal_prefill_positions(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _pos_ptr(q_pos), b, n_q, n_kv, hq, hkv, d,
        int(pretrained_window), int(local_window), float(rope_base), _schedule_id(schedule), float(softmax_scale),
        _ptr(workspace), nbytes, _stream(stream)))


def jl_plain_prefill_positions(q, k, v, out, lse, q_pos, softmax_scale=0.0, stream=None):
    b, n_q, hq, d = q.shape
    n_kv, hkv = k.shape[1], k.shape[2]
    _check(load_library().jl_plain_prefill_positions(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                                     _pos_ptr(q_pos), b, n_q, n_kv, hq, hkv, d, float(softmax_scale),
                                                     _stream(stream)))


def _table_ptr(t):
    import torch
    if t.dtype != torch.int32:
        raise TypeError("block_table must be an int32 device tensor")
    return _ptr(t)


def jl_bifocal_decode_paged(q, k_pages, v_pages, out, lse, block_table, seq_lens, pretrained_window, local_window,
                            rope_base, workspace, schedule="grouped", softmax_scale=0.0, stream=None):
    """q [B, 1, Hq, D]; page pools [n_pages, page_size, Hkv, D]; block_table int32
    [B, pages_per_seq] and seq_lens int32 [B] on the device; workspace as for
    jl_bifocal_decode with n_kv = pages_per_seq * page_size."""
    b, _, hq, d = q.shape
    n_pages, page_size, hkv = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    pages_per_seq = block_table.shape[1]
    nbytes = workspace.numel() * workspace.element_size()
    _check(load_library().jl_bifocal_decode_paged(
        _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(out), _ptr(lse), _table_ptr(block_table), _seq_lens_ptr(seq_lens),
        b, n_pages, page_size, pages_per_seq, hq, hkv, d, int(pretrained_window), int(local_window), float(rope_base),
        _schedule_id(schedule), float(softmax_scale), _ptr(workspace), nbytes, _stream(stream)))


def jl_plain_decode_paged(q, k_pages, v_pages, out, lse, block_table, seq_lens, workspace, softmax_scale=0.0,
                          stream=None):
    b, _, hq, d = q.shape
    n_pages, page_size, hkv = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    pages_per_seq = block_table.shape[1]
    nbytes = workspace.numel() * workspace.element_size()
    _check(load_library().jl_plain_decode_paged(
        _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(out), _ptr(lse), _table_ptr(block_table), _seq_lens_ptr(seq_lens),
        b, n_pages, page_size, pages_per_seq, hq, hkv, d, float(softmax_scale), _ptr(workspace), nbytes,
        _stream(stream)))
