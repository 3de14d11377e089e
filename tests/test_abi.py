"""CPU checks of the C ABI: the library loads, exports every function that
include/swgqa.h declares, and its host-only entry points behave (no kernel is
launched here)."""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np

import oracle
import sliding_window_gqa_02_amd as sw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "swgqa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(swgqa_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    names = declared_functions()
    assert names == sorted(sw.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = sw.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert isinstance(getattr(lib, name), ctypes._CFuncPtr)


def test_struct_layout():
    assert ctypes.sizeof(sw.Params) == 20 * 4
    assert ctypes.sizeof(sw.PlanEntry) == 64


def test_resident_length_and_rollback_match_oracle():
    rng = np.random.default_rng(3)
    for _ in range(3000):
        C = int(rng.integers(1, 5000))
        W = int(rng.integers(1, C + 1))
        T = int(rng.integers(0, 100_000))
        assert sw.resident_length(T, C, W) == oracle.resident_length(T, C, W)
        k = int(rng.integers(0, min(T, 40) + 1))
        assert sw.rollback_exact(T, k, C, W) == oracle.rollback_exact(T, k, C, W)
    assert sw.resident_length(5, 3, 4) == -1   # C < W
    assert sw.resident_length(5, 3, 0) == -1   # W < 1
    assert not sw.rollback_exact(5, 6, 8, 4)   # k > T


def test_resident_length_full_32bit_range_matches_oracle():
    """The library computes L(T) with a multiply-shift division by the gap
    G = C - W + 1; pin it to the oracle's plain integer division over the
    whole range a step can see (T <= 2^31, C < 2^31), powers of two and
    their neighbours for G included."""
    rng = np.random.default_rng(11)
    top = 2**31 - 1
    cases = []
    for _ in range(20000):
        C = int(rng.integers(1, top + 1))
        W = int(rng.integers(1, C + 1))
        T = int(rng.integers(0, 2**31 + 1))
        cases.append((T, C, W))
    for k in range(31):
        for G in (2**k - 1, 2**k, 2**k + 1):
            if not 1 <= G <= top:
                continue
            C = int(rng.integers(G, top + 1))
            W = C - G + 1
            for T in (0, C, C + 1, C + G, C + G + 1, 2**31, int(rng.integers(C, 2**31 + 1))):
                cases.append((T, C, W))
    cases += [(2**31, top, 1), (2**31, top, top), (2**31 - 5, 7, 7), (123456789, 1, 1)]
    for T, C, W in cases:
        assert sw.resident_length(T, C, W) == oracle.resident_length(T, C, W), (T, C, W)


def test_workspace_size():
    p = sw.make_params(32, 1, 32, 8, 128, 4608, 4096, 40000, sw.BF16)
    n = sw.workspace_size(p)
    assert n >= 256 and n % 256 == 0
    bad = sw.make_params(1, 1, 3, 2, 8, 6, 4, 8)
    assert sw.workspace_size(bad) == 0
    assert sw.workspace_size(sw.make_params(1, 1, 2, 2, 12, 6, 4, 8)) == 0


def test_workspace_holds_the_split_stash():
    """Multi-token 16-bit steps with key splits over one query tile per slice
    reserve, per (item, KV head, split, K|V), the step's largest shift in rows
    -- a multiple of the gap G = C - W + 1 no larger than G - 1 + S, at most
    64 -- and nothing once G exceeds 64; the fp32 step (same kernel, same
    partials) reserves none."""
    def extra_rows(S, C, W):
        f16 = sw.workspace_size(sw.make_params(4, S, 32, 8, 128, C, W, C + 100, sw.F16))
        f32 = sw.workspace_size(sw.make_params(4, S, 32, 8, 128, C, W, C + 100, sw.F32))
        assert f16 > 0 and f32 > 0
        rows, rem = divmod(f16 - f32, 4 * 8 * 2 * 128 * 2)
        assert rem == 0
        return rows
    for S, C, most in [(32, 1032, 36), (8, 1032, 9), (32, 1087, 64), (16, 1024, 16)]:
        rows = extra_rows(S, C, 1024)
        assert rows > 0 and rows % most == 0, (S, C, rows)
    assert extra_rows(32, 1088, 1024) == 0  # G = 65


def test_host_validation_without_gpu():
    lib = sw.load()
    buf = np.zeros(1 << 12, np.float32)
    ptr = buf.ctypes.data
    seq = np.zeros(1, np.int32).ctypes.data

    def call(p, past=ptr, present=ptr, ws_bytes=4096):
        return lib.swgqa_forward(ctypes.byref(p), ptr, ptr, ptr, past, past, seq, None, None,
                                 None, None, None,
                                 ptr, present, present, ptr, ws_bytes, None)

    assert call(sw.make_params(1, 1, 3, 2, 8, 6, 4, 8)) == sw.ERR_ARG
    assert call(sw.make_params(1, 1, 2, 2, 8, 6, 7, 8)) == sw.ERR_ARG
    assert call(sw.make_params(1, 1, 2, 2, 8, 6, -1, 8)) == sw.ERR_ARG
    assert call(sw.make_params(1, 1, 2, 2, 8, 6, 4, 8, dtype=7)) == sw.ERR_UNSUPPORTED
    assert call(sw.make_params(1, 1, 2, 2, 24, 6, 4, 8)) == sw.ERR_UNSUPPORTED
    assert call(sw.make_params(0, 1, 2, 2, 8, 6, 4, 8)) == sw.OK   # empty batch
    p = sw.make_params(1, 1, 2, 2, 8, 6, 4, 8)
    assert call(p, past=ptr + 64, present=ptr + 128) == sw.ERR_ALIAS
    assert call(p, ws_bytes=8) == sw.ERR_ARG
    assert call(sw.make_params(1, 1, 2, 2, 8, 6, 4, 8, smooth_softmax=2)) == sw.ERR_ARG
    # rotary: flags are 0/1, the caches need rows, D must be even, and the
    # caches must be given (checked before any launch)
    assert call(sw.make_params(1, 1, 2, 2, 8, 6, 4, 8, do_rotary=2, rotary_cache_rows=8)) == sw.ERR_ARG
    assert call(sw.make_params(1, 1, 2, 2, 8, 6, 4, 8, do_rotary=1, rotary_cache_rows=0)) == sw.ERR_ARG
    assert call(sw.make_params(1, 1, 2, 2, 8, 6, 4, 8, do_rotary=1, rotary_cache_rows=8,
                               rotary_interleaved=3)) == sw.ERR_ARG
    pr = sw.make_params(1, 1, 2, 2, 8, 6, 4, 8, do_rotary=1, rotary_cache_rows=8)
    need = lib.swgqa_workspace_size(ctypes.byref(pr))
    assert need > lib.swgqa_workspace_size(ctypes.byref(p))  # rotated rows + lengths
    assert call(pr, ws_bytes=need - 1) == sw.ERR_ARG
    assert call(pr, ws_bytes=need) == sw.ERR_ARG           # no cos/sin caches
    assert lib.swgqa_plan(ctypes.byref(sw.make_params(1, 1, 3, 2, 8, 6, 4, 8)), ptr, ptr, None) == sw.ERR_ARG
    for s in range(7):
        assert sw.status_string(s)


def test_eight_bit_cache_step_limits():
    """8-bit caches: steps of up to 16 tokens run on the 8-bit staged kernel
    (its LDS holds 16 quantized new rows); longer steps need the matrix-core
    kernel, whose rows are at most 512 bytes, so fp32 at head size 256 with
    more than 16 tokens is rejected before any launch -- for both code
    types; fp16 / bf16 at head size 256 take the matrix-core kernel."""
    lib = sw.load()
    buf = np.zeros(1 << 12, np.float32)
    ptr = buf.ctypes.data
    seq = np.zeros(1, np.int32).ctypes.data
    for ct in (1, 2):
        def params(S, dtype, D=256):
            return sw.make_params(1, S, 4, 2, D, 64, 32, 64, dtype, kv_cache_type=ct,
                                  k_scale=0.05, v_scale=0.04)
        assert sw.workspace_size(params(16, sw.F32)) > 0
        for S in (17, 32, 64):
            p = params(S, sw.F32)
            assert sw.workspace_size(p) == 0
            assert lib.swgqa_forward(ctypes.byref(p), ptr, ptr, ptr, ptr, ptr, seq, None, None,
                                     None, None, None, ptr, ptr, ptr, ptr, 1 << 14,
                                     None) == sw.ERR_UNSUPPORTED
            assert sw.workspace_size(params(S, sw.F16)) > 0
            assert sw.workspace_size(params(S, sw.BF16)) > 0
            assert sw.workspace_size(params(S, sw.F32, D=128)) > 0


def test_noalloc_refuses_oversized_steps_without_gpu():
    """swgqa_forward_noalloc validates and sizes the step before touching the
    device: a step needing more than its 32 MiB scratch (rotated rows of a
    long prefill) returns SWGQA_ERR_SCRATCH, invalid parameters their usual
    code."""
    lib = sw.load()
    buf = np.zeros(1 << 12, np.float32)
    ptr = buf.ctypes.data
    seq = np.zeros(8, np.int32).ctypes.data
    p = sw.make_params(8, 1024, 32, 8, 128, 2048, 1024, 1024, sw.BF16, do_rotary=1,
                       rotary_cache_rows=2048)
    assert sw.workspace_size(p) > 32 << 20

    def call(p):
        return lib.swgqa_forward_noalloc(ctypes.byref(p), ptr, ptr, ptr, ptr, ptr, seq, None,
                                         None, ptr, ptr, None, ptr, ptr, ptr, None, None)

    assert call(p) == sw.ERR_SCRATCH
    assert call(sw.make_params(1, 1, 3, 2, 8, 6, 4, 8)) == sw.ERR_ARG
    assert call(sw.make_params(0, 1, 2, 2, 8, 6, 4, 8)) == sw.OK
