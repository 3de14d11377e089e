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


def format_ulp(x: np.ndarray, dtype) -> np.ndarray:
    """Spacing of the output format at |x| (one unit in the last place)."""
    mant = {synth.F32: 23, synth.F16: 10, synth.BF16: 7}[dtype]
    emin = {synth.F32: -126, synth.F16: -14, synth.BF16: -126}[dtype]
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, emin)
    return np.ldexp(1.0, (e - mant).astype(np.int64))


def assert_outputs_close(got, ref, dtype, what=""):
    """|gpu - oracle| <= tol * max(1, |oracle|), or the two stored values are
    neighbours in the output format: each side rounds its own result (fp32 on
    the GPU, fp64 in the oracle) to nearest-even, and where the exact value
    sits near a rounding boundary the two land one ulp apart -- for bf16 one
    ulp is up to 2^-7 relative, more than the 2e-3 bound itself."""
    g = as_f64(got, dtype)
    r = as_f64(ref, dtype)
    assert not np.isnan(g).any(), f"{what}: NaN in GPU output"
    diff = np.abs(g - r)
    err = diff / np.maximum(1.0, np.abs(r))
    ok = (err <= TOL[dtype]) | (diff <= format_ulp(np.maximum(np.abs(g), np.abs(r)), dtype))
    worst = float(np.where(ok, np.minimum(err, TOL[dtype]), err).max()) if err.size else 0.0
    assert ok.all(), f"{what}: max scaled error {float(err[~ok].max()):.3g} > {TOL[dtype]} and > 1 ulp"
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
             q=None, k=None, v=None, position_ids=None):
        cfg = self.cfg
        # with rotary the cache holds rotated keys, not the generator's rows
        check_regen = check_regen and cfg.rotary < 0 and not cfg.quantized
        P = np.asarray(P, dtype=np.int64)
        if q is None:
            q, k, v = step_inputs(cfg, self.syn, P, S, self.vers)
        seq = (P + S - 1).astype(np.int32)
        st_g, out_g = self.gpu.step(S, seq, q, k, v, bias=bias, total=total, bias_bcast=bias_bcast,
                                    position_ids=position_ids)
        st_o, out_o, plan = self.ora.step(S, seq, q, k, v, bias=bias, total=total,
                                          bias_bcast=bias_bcast, position_ids=position_ids)
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
            if cfg.quantized:
                assert (gk[b, :, first_poisoned:] == cfg.poison_code).all(), what + " wrote beyond the resident range"
            else:
                rest = as_f64(gk[b, :, first_poisoned:], cfg.dtype)
                assert np.isnan(rest).all(), what + " wrote beyond the resident range"
        assert self.gpu.intact(), what + " canary overwritten"
        assert self.gpu.counters_zero(), what + " a slice counter was left non-zero"
        self.steps += 1
        return out_g, out_o, plan
