"""Python access to the CPU oracle (oracle/swgqa_oracle.cpp).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the library.  The oracle is plain C++
built with g++; it takes host numpy arrays and shares no code with the HIP
library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "swgqa_oracle.cpp")
_LIB = os.path.join(_HERE, "libswgqa_oracle.so")
_lib = None

F32, F16, BF16 = 0, 1, 2
PLAN_FIELDS = ("T", "P", "Lb", "La", "kept", "shift", "first", "hazard")


def build(force: bool = True, sanitize: bool = False, out: str | None = None) -> str:
    """Compile the oracle with g++ (optionally under ASan/UBSan)."""
    target = out or _LIB
    if force or not os.path.exists(target):
        cmd = ["g++", "-std=c++17", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-fopenmp",
               "-Wall", "-Wextra"]
        if sanitize:
            cmd += ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", "-g"]
        tmp = target + ".tmp%d" % os.getpid()
        subprocess.check_call(cmd + ["-o", tmp, _SRC])
        os.replace(tmp, target)
    return target


class Params(ctypes.Structure):
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


def lib():
    """The loaded oracle library: libswgqa_oracle.so next to this file, or
    the build named by SWGQA_ORACLE_LIB (e.g. one built with sanitize=True)."""
    global _lib
    if _lib is None:
        path = os.environ.get("SWGQA_ORACLE_LIB", _LIB)
        if not os.path.exists(path):
            build(force=False, out=path)
        L = ctypes.CDLL(path)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        L.swgqa_oracle_resident_length.restype = i64
        L.swgqa_oracle_resident_length.argtypes = [i64, i64, i64]
        L.swgqa_oracle_resident_lengths.restype = None
        L.swgqa_oracle_resident_lengths.argtypes = [vp, i64, i64, i64, vp]
        L.swgqa_oracle_rollback_exact.restype = ctypes.c_int
        L.swgqa_oracle_rollback_exact.argtypes = [i64, i64, i64, i64]
        L.swgqa_oracle_plan.restype = ctypes.c_int
        L.swgqa_oracle_plan.argtypes = [ctypes.POINTER(Params), vp, vp]
        L.swgqa_oracle_forward.restype = ctypes.c_int
        L.swgqa_oracle_forward.argtypes = [ctypes.POINTER(Params)] + [vp] * 15
        L.swgqa_oracle_forward_compact_first.restype = ctypes.c_int
        L.swgqa_oracle_forward_compact_first.argtypes = [ctypes.POINTER(Params)] + [vp] * 9
        L.swgqa_oracle_decode.restype = ctypes.c_double
        L.swgqa_oracle_decode.argtypes = [i32, ctypes.c_uint32]
        L.swgqa_oracle_encode.restype = ctypes.c_uint32
        L.swgqa_oracle_encode.argtypes = [i32, ctypes.c_double]
        L.swgqa_oracle_quantize_e4m3.restype = ctypes.c_uint32
        L.swgqa_oracle_quantize_e4m3.argtypes = [ctypes.c_double, ctypes.c_float]
        L.swgqa_oracle_decode_e4m3.restype = ctypes.c_double
        L.swgqa_oracle_decode_e4m3.argtypes = [ctypes.c_uint32]
        L.swgqa_oracle_set_threads.restype = ctypes.c_int
        L.swgqa_oracle_set_threads.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def make_params(B, S, Hq, Hkv, D, C, W, total, dtype=F32, scale=0.0,
                softcap=0.0, bias_batch=1, bias_heads=1, smooth_softmax=0,
                do_rotary=0, rotary_interleaved=0, rotary_cache_rows=0, kv_cache_type=0,
                k_scale=0.0, v_scale=0.0) -> Params:
    return Params(B, S, Hq, Hkv, D, C, W, total, scale, softcap, dtype,
                  bias_batch, bias_heads, smooth_softmax, do_rotary, rotary_interleaved,
                  rotary_cache_rows, kv_cache_type, k_scale, v_scale)


def _ptr(a):
    return None if a is None else a.ctypes.data


def resident_length(T: int, C: int, W: int) -> int:
    return lib().swgqa_oracle_resident_length(T, C, W)


def resident_lengths(T: np.ndarray, C: int, W: int) -> np.ndarray:
    T = np.ascontiguousarray(T, dtype=np.int64)
    out = np.empty_like(T)
    lib().swgqa_oracle_resident_lengths(T.ctypes.data, T.size, C, W, out.ctypes.data)
    return out


def rollback_exact(T: int, k: int, C: int, W: int) -> bool:
    return bool(lib().swgqa_oracle_rollback_exact(T, k, C, W))


def plan(p: Params, seqlens_k: np.ndarray):
    seqlens_k = np.ascontiguousarray(seqlens_k, dtype=np.int32)
    out = np.zeros((p.batch_size, 8), dtype=np.int64)
    st = lib().swgqa_oracle_plan(ctypes.byref(p), _ptr(seqlens_k), _ptr(out))
    return st, out


def forward(p: Params, query, key, value, past_key, past_value, seqlens_k,
            bias=None, present_key=None, present_value=None, output=None, head_sink=None,
            cos_cache=None, sin_cache=None, position_ids=None):
    """Runs one step.  present_* default to past_* (in place: the arrays are
    modified).  Returns (status, output, plan)."""
    seqlens_k = np.ascontiguousarray(seqlens_k, dtype=np.int32)
    for a in (query, key, value, past_key, past_value):
        assert a.flags.c_contiguous
    if present_key is None:
        present_key = past_key
    if present_value is None:
        present_value = past_value
    if output is None:
        output = np.empty_like(query)
    planbuf = np.zeros((p.batch_size, 8), dtype=np.int64)
    if position_ids is not None:
        position_ids = np.ascontiguousarray(position_ids, dtype=np.int64)
    st = lib().swgqa_oracle_forward(
        ctypes.byref(p), _ptr(query), _ptr(key), _ptr(value), _ptr(past_key),
        _ptr(past_value), _ptr(seqlens_k), _ptr(bias), _ptr(head_sink), _ptr(cos_cache),
        _ptr(sin_cache), _ptr(position_ids), _ptr(output),
        _ptr(present_key), _ptr(present_value), _ptr(planbuf))
    return st, output, planbuf


def forward_compact_first(p: Params, query, key, value, cache_key, cache_value,
                          seqlens_k, bias=None, head_sink=None):
    seqlens_k = np.ascontiguousarray(seqlens_k, dtype=np.int32)
    output = np.empty_like(query)
    st = lib().swgqa_oracle_forward_compact_first(
        ctypes.byref(p), _ptr(query), _ptr(key), _ptr(value), _ptr(cache_key),
        _ptr(cache_value), _ptr(seqlens_k), _ptr(bias), _ptr(head_sink), _ptr(output))
    return st, output


def quantize_e4m3(x: float, scale: float) -> int:
    return lib().swgqa_oracle_quantize_e4m3(x, scale)


def decode_e4m3(code: int) -> float:
    return lib().swgqa_oracle_decode_e4m3(code)


def decode(dtype: int, bits: int) -> float:
    return lib().swgqa_oracle_decode(dtype, bits)


def encode(dtype: int, x: float) -> int:
    return lib().swgqa_oracle_encode(dtype, x)


def set_threads(n: int) -> int:
    return lib().swgqa_oracle_set_threads(n)
