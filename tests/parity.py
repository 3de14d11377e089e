"""Lock-step driver for the GPU parity tests: the same seeded inputs go to the
HIP path (through the C ABI) and to the CPU oracle, each of which advances
its own cache; after every step the outputs are compared within tolerance and
the resident rows byte for byte (and against the layout regenerated from
absolute positions).
"""
from __future__ import annotations

import sys

import numpy as np

import oracle
import synth
from tests.scenario import Cfg, OracleBackend, Versions, as_f64, layout_rows, step_inputs

TOL = {synth.F32: 1e-5, synth.F16: 2e-3, synth.BF16: 2e-3}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def assert_outputs_close(got, ref, dtype, what=""):
    g = as_f64(got, dtype)
    r = as_f64(ref, dtype)
    assert not np.isnan(g).any(), f"{what}: NaN in GPU output"
    err = np.abs(g - r) / np.maximum(1.0, np.abs(r))
    worst = float(err.max()) if err.size else 0.0
    assert worst <= TOL[dtype], f"{what}: max scaled error {worst:.3g} > {TOL[dtype]}"
    return worst


def assert_rows_equal(gpu_cache, ora_cache, b, L, what=""):
    g = np.ascontiguousarray(gpu_cache[b, :, :L]).view(np.uint8)
    o = np.ascontiguousarray(ora_cache[b, :, :L]).view(np.uint8)
    assert np.array_equal(g, o), f"{what}: present rows [0,{L}) differ for item {b}"


class Lockstep:
    def __init__(self, cfg: Cfg, mode="shared", K=None, V=None, B=None, vers=None):
        from tests.gpu_backend import GpuBackend
        self.cfg = cfg
        self.B = cfg.B if B is None else B
        self.syn = cfg.synth()
        self.vers = vers or Versions(self.B)
        self.gpu = GpuBackend(cfg, K, V, B=self.B, mode=mode)
        self.ora = OracleBackend(cfg, K, V, B=self.B)
        self.worst = 0.0
        self.steps = 0

    def step(self, P, S, bias=None, total=None, bias_bcast=(1, 1), check_regen=True,
             q=None, k=None, v=None):
        cfg = self.cfg
        P = np.asarray(P, dtype=np.int64)
        if q is None:
            q, k, v = step_inputs(cfg, self.syn, P, S, self.vers)
        seq = (P + S - 1).astype(np.int32)
        st_g, out_g = self.gpu.step(S, seq, q, k, v, bias=bias, total=total, bias_bcast=bias_bcast)
        st_o, out_o, plan = self.ora.step(S, seq, q, k, v, bias=bias, total=total, bias_bcast=bias_bcast)
        what = f"step {self.steps} S={S} P={list(P[:4])}"
        assert st_o == 0, what
        assert st_g == 0, what
        self.worst = max(self.worst, assert_outputs_close(out_g, out_o, cfg.dtype, what))
        gk, gv = self.gpu.present_host()
        for b in range(len(P)):
            La = int(plan[b, 3])
            assert_rows_equal(gk, self.ora.K, b, La, what + " K")
            assert_rows_equal(gv, self.ora.V, b, La, what + " V")
            if check_regen:
                L, rk, rv = layout_rows(cfg, self.syn, b, int(P[b]) + S, self.vers)
                assert L == La
                assert np.array_equal(np.ascontiguousarray(gk[b, :, :L]).view(np.uint8), rk.view(np.uint8)), what
                assert np.array_equal(np.ascontiguousarray(gv[b, :, :L]).view(np.uint8), rv.view(np.uint8)), what
            # this implementation writes only rows [0, La): rows that were
            # poisoned before the step ([Lb, C) in place, all of a separate
            # present buffer) stay NaN beyond La
            first_poisoned = max(La, int(plan[b, 2])) if self.gpu.mode == "shared" else La
            rest = as_f64(gk[b, :, first_poisoned:], cfg.dtype)
            assert np.isnan(rest).all(), what + " wrote beyond the resident range"
        assert self.gpu.intact(), what + " canary overwritten"
        self.steps += 1
        return out_g, out_o, plan
