"""Python binding of libswgqa: one GroupQueryAttention step over a windowed
KV cache on AMD MI355X (gfx950).

Argument marshalling only -- every step of the computation runs in the HIP
kernels of libswgqa.so (built from csrc/ by build.py).  Tensors are torch
tensors on the GPU; PyTorch provides device memory and streams.  There is no
CPU fallback: if the library cannot be loaded, importing the binding's entry
points raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libswgqa.so")

F32, F16, BF16 = 0, 1, 2
OK, ERR_ARG, ERR_UNSUPPORTED, ERR_ALIAS, ERR_DEVICE_INPUT, ERR_HIP, ERR_SCRATCH = range(7)

# Symbols declared in include/swgqa.h.
EXPORTS = (
    "swgqa_workspace_size", "swgqa_workspace_init", "swgqa_forward", "swgqa_forward_noalloc",
    "swgqa_plan",
    "swgqa_resident_length", "swgqa_rollback_exact", "swgqa_device_status",
    "swgqa_status_string",
)


class SwgqaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


class Params(ctypes.Structure):
    """Mirror of swgqa_params."""
    _fields_ = [
        ("batch_size", ctypes.c_int32),
        ("sequence_length", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("kv_num_heads", ctypes.c_int32),
        ("head_size", ctypes.c_int32),
        ("capacity", ctypes.c_int32),
        ("local_window_size", ctypes.c_int32),
        ("total_sequence_length", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("softcap", ctypes.c_float),
        ("dtype", ctypes.c_int32),
        ("bias_dim0_is_batch", ctypes.c_int32),
        ("bias_dim1_is_heads", ctypes.c_int32),
        ("smooth_softmax", ctypes.c_int32),
        ("do_rotary", ctypes.c_int32),
        ("rotary_interleaved", ctypes.c_int32),
        ("rotary_cache_rows", ctypes.c_int32),
        ("kv_cache_type", ctypes.c_int32),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
    ]


class PlanEntry(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in
                ("T", "P", "Lb", "La", "kept", "shift", "first", "hazard")]


_lib = None


def load(path: str = LIB_PATH):
    """Loads libswgqa.so (building it first only if it does not exist)."""
    global _lib
    if _lib is not None:
        return _lib
    # torch ships its own HIP runtime under the same soname; importing it
    # first makes this library bind to that runtime, so that torch's streams
    # and allocations are valid handles here.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(path):
        from . import build as _build
        _build.build()
    L = ctypes.CDLL(path)
    vp, sz, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64
    P = ctypes.POINTER(Params)
    L.swgqa_workspace_size.restype = sz
    L.swgqa_workspace_size.argtypes = [P]
    L.swgqa_workspace_init.restype = ctypes.c_int
    L.swgqa_workspace_init.argtypes = [vp, sz, vp]
    L.swgqa_forward.restype = ctypes.c_int
    L.swgqa_forward.argtypes = [P] + [vp] * 15 + [sz, vp]
    L.swgqa_forward_noalloc.restype = ctypes.c_int
    L.swgqa_forward_noalloc.argtypes = [P] + [vp] * 16
    L.swgqa_plan.restype = ctypes.c_int
    L.swgqa_plan.argtypes = [P, vp, vp, vp]
    L.swgqa_resident_length.restype = i64
    L.swgqa_resident_length.argtypes = [i64, i64, i64]
    L.swgqa_rollback_exact.restype = ctypes.c_int
    L.swgqa_rollback_exact.argtypes = [i64, i64, i64, i64]
    L.swgqa_device_status.restype = ctypes.c_int
    L.swgqa_device_status.argtypes = [vp, ctypes.c_int, vp]
    L.swgqa_status_string.restype = ctypes.c_char_p
    L.swgqa_status_string.argtypes = [ctypes.c_int]
    _lib = L
    return L


def status_string(status: int) -> str:
    return load().swgqa_status_string(status).decode()


def make_params(batch_size, sequence_length, num_heads, kv_num_heads, head_size,
                capacity, local_window_size, total_sequence_length, dtype=F32,
                scale=0.0, softcap=0.0, bias_dim0_is_batch=1,
                bias_dim1_is_heads=1, smooth_softmax=0, do_rotary=0, rotary_interleaved=0,
                rotary_cache_rows=0, kv_cache_type=0, k_scale=0.0, v_scale=0.0) -> Params:
    return Params(batch_size, sequence_length, num_heads, kv_num_heads, head_size,
                  capacity, local_window_size, total_sequence_length, scale, softcap,
                  dtype, bias_dim0_is_batch, bias_dim1_is_heads, smooth_softmax, do_rotary,
                  rotary_interleaved, rotary_cache_rows, kv_cache_type, k_scale, v_scale)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def workspace_size(p: Params) -> int:
    return load().swgqa_workspace_size(ctypes.byref(p))


def workspace_init(workspace, stream=None) -> None:
    st = load().swgqa_workspace_init(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream(stream))
    if st != OK:
        raise SwgqaError(st, "swgqa_workspace_init")


def forward(p: Params, query, key, value, past_key, past_value, seqlens_k,
            attention_bias, output, present_key, present_value, workspace,
            stream=None, head_sink=None, cos_cache=None, sin_cache=None,
            position_ids=None) -> None:
    """Enqueues one step (see include/swgqa.h).  All tensors on the GPU."""
    st = load().swgqa_forward(
        ctypes.byref(p), _ptr(query), _ptr(key), _ptr(value), _ptr(past_key),
        _ptr(past_value), _ptr(seqlens_k), _ptr(attention_bias), _ptr(head_sink),
        _ptr(cos_cache), _ptr(sin_cache), _ptr(position_ids), _ptr(output),
        _ptr(present_key), _ptr(present_value), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    if st != OK:
        raise SwgqaError(st, "swgqa_forward")


def forward_status(p: Params, query, key, value, past_key, past_value, seqlens_k,
                   attention_bias, output, present_key, present_value, workspace,
                   workspace_bytes=None, stream=None, head_sink=None, cos_cache=None,
                   sin_cache=None, position_ids=None) -> int:
    """Like forward() but returns the status code instead of raising."""
    nbytes = workspace.numel() * workspace.element_size() if workspace_bytes is None \
        else workspace_bytes
    return load().swgqa_forward(
        ctypes.byref(p), _ptr(query), _ptr(key), _ptr(value), _ptr(past_key),
        _ptr(past_value), _ptr(seqlens_k), _ptr(attention_bias), _ptr(head_sink),
        _ptr(cos_cache), _ptr(sin_cache), _ptr(position_ids),
        _ptr(output), _ptr(present_key), _ptr(present_value), _ptr(workspace), nbytes,
        _stream(stream))


def forward_noalloc_status(p: Params, query, key, value, past_key, past_value, seqlens_k,
                           attention_bias, output, present_key, present_value,
                           device_status=None, stream=None, head_sink=None, cos_cache=None,
                           sin_cache=None, position_ids=None) -> int:
    """One step through swgqa_forward_noalloc (the library's static scratch
    as workspace); returns the status code.  device_status: None or an int32
    device tensor of one element receiving device item errors."""
    return load().swgqa_forward_noalloc(
        ctypes.byref(p), _ptr(query), _ptr(key), _ptr(value), _ptr(past_key),
        _ptr(past_value), _ptr(seqlens_k), _ptr(attention_bias), _ptr(head_sink),
        _ptr(cos_cache), _ptr(sin_cache), _ptr(position_ids),
        _ptr(output), _ptr(present_key), _ptr(present_value), _ptr(device_status),
        _stream(stream))


def plan(p: Params, seqlens_k, plan_out, stream=None) -> None:
    st = load().swgqa_plan(ctypes.byref(p), _ptr(seqlens_k), _ptr(plan_out), _stream(stream))
    if st != OK:
        raise SwgqaError(st, "swgqa_plan")


def resident_length(T: int, C: int, W: int) -> int:
    return load().swgqa_resident_length(T, C, W)


def rollback_exact(T: int, k: int, C: int, W: int) -> bool:
    return bool(load().swgqa_rollback_exact(T, k, C, W))


def device_status(workspace, clear: bool = False, stream=None) -> int:
    return load().swgqa_device_status(_ptr(workspace), 1 if clear else 0, _stream(stream))
