"""Seeded synthetic inputs for windowed GQA steps.

Every value is a pure function of a key ``(seed, tensor, b, head, pos, d,
version)``: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014) hashes the key, and the Box-Muller transform
turns two 24-bit uniforms into two N(0, 1) samples (synth_core.c, a small C
library of its own, built with gcc).  Because a K/V row is
keyed by its *absolute* position, the expected contents of any cache layout
can be regenerated from positions alone, without running any attention code.

Values are computed in float64, rounded to float32, then rounded to
nearest-even into the step's element type.  This module holds none of the
attention or cache arithmetic; it only produces inputs, and it is shared by
the tests, the benchmark and the smoke check.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

# Tensor tags of the key.
Q, K, V, BIAS = 0, 1, 2, 3

F32, F16, BF16 = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth_core.c")
_LIB = os.path.join(_HERE, "libsynth.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the generator core with the host C compiler (gcc)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _core():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        lib.synth_normal_rows.restype = None
        lib.synth_normal_rows.argtypes = [
            ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int32, ctypes.c_double, ctypes.c_void_p]
        _lib = lib
    return _lib


def normal_rows(seed, tensor, b, head, pos, version, n: int,
                std: float = 1.0) -> np.ndarray:
    """float32 N(0, std^2) samples, shape broadcast(b, head, pos, version) + (n,).

    Element ``d`` of a row is the key's d-th sample; every row is independent
    of every other, so any subset of rows can be regenerated on its own.
    """
    b, head, pos, version = np.broadcast_arrays(
        np.asarray(b), np.asarray(head), np.asarray(pos), np.asarray(version))
    shape = b.shape
    cols = [np.ascontiguousarray(a, dtype=np.int64).reshape(-1)
            for a in (b, head, pos, version)]
    nrows = cols[0].shape[0]
    out = np.empty((nrows, n), dtype=np.float32)
    if nrows and n:
        _core().synth_normal_rows(
            ctypes.c_uint64(seed & 0xFFFFFFFFFFFFFFFF), tensor, nrows,
            *[c.ctypes.data for c in cols], n, float(std), out.ctypes.data)
    return out.reshape(shape + (n,))


def to_storage(x: np.ndarray, dtype: int) -> np.ndarray:
    """Round float32 values to the element type, returned as storage:
    float32 for fp32, uint16 bit patterns for fp16 / bf16 (nearest-even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == F32:
        return x
    if dtype == F16:
        return x.astype(np.float16).view(np.uint16)
    if dtype == BF16:
        u = x.view(np.uint32)
        r = (u >> np.uint32(16)) & np.uint32(1)
        r += np.uint32(0x7FFF)
        r += u                      # no wrap: only NaNs lie above 0xFFFF8000
        r >>= np.uint32(16)
        return r.astype(np.uint16)
    raise ValueError(f"unknown dtype {dtype}")


def from_storage(a: np.ndarray, dtype: int) -> np.ndarray:
    """Storage (as produced by to_storage) back to float64 values."""
    if dtype == F32:
        return a.astype(np.float64)
    if dtype == F16:
        return a.view(np.float16).astype(np.float64)
    if dtype == BF16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype}")


def storage_dtype(dtype: int):
    return np.float32 if dtype == F32 else np.uint16


def elem_bytes(dtype: int) -> int:
    return 4 if dtype == F32 else 2


def rotary_tables(rows: int, head_size: int, dtype: int, base: float = 10000.0):
    """cos / sin tables (rows, head_size / 2) in storage form: row pos, column
    k holds cos / sin of pos * base^(-2k / head_size), computed in float64
    and rounded once to the element type (the usual frequency ladder)."""
    k = np.arange(head_size // 2)
    ang = np.arange(rows)[:, None] * base ** (-2.0 * k[None, :] / head_size)
    return to_storage(np.cos(ang), dtype), to_storage(np.sin(ang), dtype)


class Synth:
    """Generator bound to one seed, head counts and element type.

    ``version`` lets a caller re-draw a position (a rejected draft token that
    is later appended again with different contents); it is an int array
    broadcastable to the rows requested.
    """

    def __init__(self, seed: int, num_heads: int, kv_num_heads: int,
                 head_size: int, dtype: int, v_pos_in_elem0: bool = False,
                 zero_query: bool = False, bias_std: float = 0.1):
        self.seed = seed
        self.Hq = num_heads
        self.Hkv = kv_num_heads
        self.D = head_size
        self.dtype = dtype
        self.v_pos_in_elem0 = v_pos_in_elem0
        self.zero_query = zero_query
        self.bias_std = bias_std

    # -- rows keyed by absolute position ------------------------------------
    def kv_rows(self, tensor: int, b, head, pos, version=0) -> np.ndarray:
        x = normal_rows(self.seed, tensor, b, head, pos, version, self.D)
        if tensor == V and self.v_pos_in_elem0:
            x[..., 0] = np.broadcast_to(np.asarray(pos), x.shape[:-1])
        return to_storage(x, self.dtype)

    def q_rows(self, b, head, pos, version=0) -> np.ndarray:
        x = normal_rows(self.seed, Q, b, head, pos, version, self.D)
        if self.zero_query:
            x[...] = 0.0
        return to_storage(x, self.dtype)

    # -- whole step inputs --------------------------------------------------
    def step_inputs(self, P: np.ndarray, S: int, version=None):
        """query (B,S,Hq*D), key/value (B,S,Hkv*D) for items starting at P[b]."""
        P = np.asarray(P, dtype=np.int64)
        B = P.shape[0]
        pos = P[:, None] + np.arange(S)[None, :]                 # (B,S)
        ver = np.zeros_like(pos) if version is None else np.asarray(version)
        bq = np.arange(B)[:, None, None]
        hq = np.arange(self.Hq)[None, None, :]
        q = self.q_rows(bq, hq, pos[:, :, None], ver[:, :, None])  # (B,S,Hq,D)
        hk = np.arange(self.Hkv)[None, None, :]
        k = self.kv_rows(K, bq, hk, pos[:, :, None], ver[:, :, None])
        v = self.kv_rows(V, bq, hk, pos[:, :, None], ver[:, :, None])
        return (q.reshape(B, S, self.Hq * self.D),
                k.reshape(B, S, self.Hkv * self.D),
                v.reshape(B, S, self.Hkv * self.D))

    def bias_f32(self, b_items, P, S: int, total: int,
                 version_of=None) -> np.ndarray:
        """attention_bias values (B, Hq, S, total) ~ N(0, bias_std^2) as
        float32, entry keyed by (b, h, absolute query position, absolute key
        position); pass through to_storage for the element type."""
        P = np.asarray(P, dtype=np.int64)
        B = P.shape[0]
        out = np.empty((B, self.Hq, S, total), dtype=np.float32)
        for bi in range(B):
            qpos = P[bi] + np.arange(S)
            ver = 0 if version_of is None else version_of(bi, qpos)
            x = normal_rows(self.seed, BIAS, b_items[bi],
                            np.arange(self.Hq)[:, None],
                            qpos[None, :], np.broadcast_to(ver, qpos.shape)[None, :],
                            total, std=self.bias_std)
            out[bi] = x
        return out

