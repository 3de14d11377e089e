"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each test names the passage it pins (page title, section).  None of these
re-types the oracle's own formula: they compare it with an independent
recurrence, brute force, closed forms, printed values, or invariants.
"""
from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
import synth
from tests.scenario import (Cfg, OracleBackend, Versions, as_f64, layout_rows,
                            nan_array, step_inputs)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# P1. Resident length vs the one-token recurrence.
# "Specify GroupQueryAttention windowed KV cache layout contract",
# Description: L(T) closed form and min(T, W) <= L(T) <= min(T, C).
# "[CPU] Add windowed kv cache for GQA", drifting layout: the append point
# grows by one per token and a whole gap of G rows is reclaimed when the
# buffer would overflow.
def _recurrence(Tmax, C, W):
    G = C - W + 1
    out = np.zeros(Tmax + 1, dtype=np.int64)
    l = 0
    for t in range(1, Tmax + 1):
        l += 1
        if l > C:
            l -= G
        out[t] = l
    return out


def test_p1_resident_length_small_all_pairs():
    Tmax = 10_000
    T = np.arange(Tmax + 1)
    for C in range(1, 65):
        # vectorised recurrence over all W for this C
        Ws = np.arange(1, C + 1)
        G = C - Ws + 1
        ref = np.zeros((Tmax + 1, C), dtype=np.int64)
        l = np.zeros(C, dtype=np.int64)
        for t in range(1, Tmax + 1):
            l += 1
            l = np.where(l > C, l - G, l)
            ref[t] = l
        for wi, W in enumerate(Ws):
            got = oracle.resident_lengths(T, C, int(W))
            assert np.array_equal(got, ref[:, wi]), (C, W)
            assert np.all(got >= np.minimum(T, W)) and np.all(got <= np.minimum(T, C))


@pytest.mark.parametrize("C,W", [(6, 4), (384, 128), (136, 128), (1032, 1024),
                                 (1055, 1024), (4608, 4096), (128, 128)])
def test_p1_resident_length_config_pairs(C, W):
    Tmax = 40_000
    T = np.arange(Tmax + 1)
    got = oracle.resident_lengths(T, C, W)
    assert np.array_equal(got, _recurrence(Tmax, C, W))
    assert np.all(got >= np.minimum(T, W)) and np.all(got <= np.minimum(T, C))
    assert np.all(np.diff(got) <= 1)
    # second closed form for T > C: L = W + ((T - C - 1) mod G)
    G = C - W + 1
    big = T[T > C]
    assert np.array_equal(got[T > C], W + ((big - C - 1) % G))


def test_p1_int64_range():
    # the planner works in int64 (PR #31142 review thread): no wrap near 2^31
    T = np.array([2**31 - 1, 2**31 + 5, 2**40 + 3], dtype=np.int64)
    C, W = 4608, 4096
    G = C - W + 1
    got = oracle.resident_lengths(T, C, W)
    assert np.array_equal(got, W + ((T - C - 1) % G))


# ---------------------------------------------------------------------------
# Element conversions used for outputs: pinned against numpy's IEEE binary16
# cast and against a brute-force nearest-even search for bf16.
def test_conversions_fp16_against_numpy():
    rng = np.random.default_rng(7)
    xs = np.concatenate([rng.normal(0, 1, 3000), rng.normal(0, 1e-5, 1000),
                         rng.normal(0, 3e4, 1000), [0.0, -0.0, 65504.0, 65520.0,
                                                     65519.99, 6e-8, 2.98e-8,
                                                     2.99e-8, 1e-9]])
    for x in xs:
        with np.errstate(over="ignore"):
            want = int(np.array([x], dtype=np.float64).astype(np.float16).view(np.uint16)[0])
        assert oracle.encode(synth.F16, float(x)) == want, x
        assert oracle.decode(synth.F16, want) == float(np.uint16(want).view(np.float16))


def test_conversions_bf16_nearest_even():
    rng = np.random.default_rng(8)
    xs = np.concatenate([rng.normal(0, 1, 2000), rng.normal(0, 1e-38, 200),
                         rng.normal(0, 1e30, 200)])
    allbits = np.arange(1 << 16, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        vals = (allbits << 16).view(np.float32).astype(np.float64)
    finite = np.isfinite(vals)
    for x in xs:
        bits = oracle.encode(synth.BF16, float(x))
        got = oracle.decode(synth.BF16, bits)
        err = abs(got - x)
        best = np.min(np.abs(vals[finite] - x))
        assert err == best, x
        if err != 0:  # ties go to the even significand
            cands = allbits[finite][np.abs(vals[finite] - x) == best]
            if len(cands) == 2:
                assert bits % 2 == 0
    assert oracle.encode(synth.BF16, 1.0 + 2**-8) == 0x3F80      # tie -> even
    assert oracle.encode(synth.BF16, 1.0 + 3 * 2**-8) == 0x3F82  # tie -> even


# ---------------------------------------------------------------------------
# Brute force: a full-length cache that never evicts, with an explicit
# causal-and-window mask.  "[CPU] Add windowed kv cache for GQA", intro:
# windowed results equal those of a full-length cache; causal rule of
# "Fix CPU Attention causal mask ..." (j <= i + past); window of W keys.
def brute_force(cfg: Cfg, syn, b, P, S, vers, q_storage, bias=None):
    T = P + S
    pos = np.arange(T)
    ver = vers.of(b, pos)[None, :]
    heads = np.arange(cfg.Hkv)[:, None]
    Kall = as_f64(syn.kv_rows(synth.K, b, heads, pos[None, :], ver), cfg.dtype)
    Vall = as_f64(syn.kv_rows(synth.V, b, heads, pos[None, :], ver), cfg.dtype)
    q = as_f64(q_storage, cfg.dtype).reshape(S, cfg.Hq, cfg.D)
    scale = cfg.scale if cfg.scale > 0 else 1.0 / np.sqrt(cfg.D)
    i = np.arange(S)[:, None]
    j = np.arange(T)[None, :]
    mask = (j <= P + i) & (j > P + i - cfg.W)
    out = np.zeros((S, cfg.Hq, cfg.D))
    grp = cfg.Hq // cfg.Hkv
    for h in range(cfg.Hq):
        g = h // grp
        s = scale * (q[:, h, :] @ Kall[g].T)
        if cfg.softcap > 0:
            s = cfg.softcap * np.tanh(s / cfg.softcap)
        if bias is not None:
            s = s + bias[h, :, :T]
        s = np.where(mask, s, -np.inf)
        w = np.exp(s - s.max(axis=1, keepdims=True))
        out[:, h, :] = (w @ Vall[g]) / w.sum(axis=1, keepdims=True)
    return out.reshape(S, cfg.Hq * cfg.D)


def _close_to_rounded(got_storage, ref, dtype):
    got = as_f64(got_storage, dtype)
    # half an ulp of the format plus fp64 noise, with the subnormal quantum
    # as the absolute floor
    rel = {synth.F32: 2.0**-23, synth.F16: 2.0**-10, synth.BF16: 2.0**-7}[dtype]
    floor = {synth.F32: 2.0**-149, synth.F16: 2.0**-24, synth.BF16: 2.0**-133}[dtype]
    return np.all(np.abs(got - ref) <= rel * np.abs(ref) + floor)


def run_sequence(cfg: Cfg, steps, check=None, vers=None, bias_fn=None):
    """Drive the oracle through `steps` (list of S) for every item in lock
    step from T=0.  Returns per-position outputs {(b, pos): row}."""
    syn = cfg.synth()
    vers = vers or Versions(cfg.B)
    be = OracleBackend(cfg)
    T = np.zeros(cfg.B, dtype=np.int64)
    outs = {}
    for S in steps:
        P = T.copy()
        T = T + S
        q, k, v = step_inputs(cfg, syn, P, S, vers)
        bias = None
        if bias_fn is not None:
            bias = bias_fn(syn, P, S, int(T.max()))
        st, out, plan = be.step(S, T - 1, q, k, v, bias=bias)
        assert st == 0
        for b in range(cfg.B):
            for i in range(S):
                outs[(b, int(P[b]) + i)] = out[b, i].copy()
        if check is not None:
            check(be, syn, P, S, T, q, out, plan, vers, bias)
    return outs, be


def _check_layout(cfg):
    def check(be, syn, P, S, T, q, out, plan, vers, bias):
        for b in range(cfg.B):
            L, k, v = layout_rows(cfg, syn, b, int(T[b]), vers)
            assert plan[b, 3] == L
            assert np.array_equal(be.K[b, :, :L].view(np.uint8), k.view(np.uint8))
            assert np.array_equal(be.V[b, :, :L].view(np.uint8), v.view(np.uint8))
    return check


# ---------------------------------------------------------------------------
# P2 + P5: layout by regeneration after every step, and outputs equal to the
# full-cache brute force, over many small shapes and step splits.
SMALL = [
    Cfg(B=1, Hq=4, Hkv=2, D=8, C=6, W=4, seed=1001, v_pos=True),
    Cfg(B=2, Hq=2, Hkv=2, D=4, C=5, W=5, seed=11),
    Cfg(B=1, Hq=3, Hkv=1, D=2, C=7, W=1, seed=12),
    Cfg(B=2, Hq=4, Hkv=1, D=8, C=9, W=3, seed=13, dtype=synth.F16),
    Cfg(B=1, Hq=2, Hkv=1, D=8, C=8, W=6, seed=14, dtype=synth.BF16, softcap=2.0),
    Cfg(B=1, Hq=4, Hkv=4, D=1, C=1, W=1, seed=15),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: f"C{c.C}W{c.W}D{c.D}t{c.dtype}")
def test_p2_p5_layout_and_brute_force(cfg):
    rng = np.random.default_rng(cfg.seed)
    steps = [int(s) for s in rng.integers(1, 2 * cfg.C + 2, size=12)]
    vers = Versions(cfg.B)
    layout = _check_layout(cfg)

    def check(be, syn, P, S, T, q, out, plan, vers_, bias):
        layout(be, syn, P, S, T, q, out, plan, vers_, bias)
        for b in range(cfg.B):
            ref = brute_force(cfg, syn, b, int(P[b]), S, vers_, q[b])
            assert _close_to_rounded(out[b], ref, cfg.dtype)

    run_sequence(cfg, steps, check=check, vers=vers)


def test_p5_brute_force_catches_a_planted_window_error():
    """The brute-force pin is sensitive: a window one key wider than the
    contract's changes the outputs (the oracle is checked against W, and a
    copy of the reference with W+1 disagrees)."""
    cfg = Cfg(B=1, Hq=2, Hkv=1, D=4, C=6, W=3, seed=3)
    outs, _ = run_sequence(cfg, [8, 1, 1])
    syn = cfg.synth()
    vers = Versions(1)
    wide = Cfg(**{**cfg.__dict__, "W": 4, "C": 6})
    q, _, _ = step_inputs(cfg, syn, np.array([9]), 1, vers)
    ref_ok = brute_force(cfg, syn, 0, 9, 1, vers, q[0])
    ref_wide = brute_force(wide, syn, 0, 9, 1, vers, q[0])
    assert _close_to_rounded(outs[(0, 9)][None], ref_ok, cfg.dtype)
    assert not _close_to_rounded(outs[(0, 9)][None], ref_wide, cfg.dtype)


# ---------------------------------------------------------------------------
# P3. Step-split invariance: "Specify ... layout contract", Description (the
# layout depends only on T; a multi-token step leaves the layout the same
# tokens leave one at a time) and Summary of Changes (8-token prefill then a
# 4-token step vs four 1-token steps, byte-identical presents and outputs).
def test_p3_prefill8_then_4_vs_four_single_steps():
    cfg = Cfg(B=1, Hq=4, Hkv=2, D=8, C=6, W=4, seed=1001, v_pos=True)
    outs_a, be_a = run_sequence(cfg, [8, 4], check=_check_layout(cfg))
    outs_b, be_b = run_sequence(cfg, [8, 1, 1, 1, 1], check=_check_layout(cfg))
    L = oracle.resident_length(12, cfg.C, cfg.W)
    assert np.array_equal(be_a.K[:, :, :L].view(np.uint8), be_b.K[:, :, :L].view(np.uint8))
    assert np.array_equal(be_a.V[:, :, :L].view(np.uint8), be_b.V[:, :, :L].view(np.uint8))
    for pos in range(12):
        assert np.array_equal(outs_a[(0, pos)].view(np.uint8), outs_b[(0, pos)].view(np.uint8))


@pytest.mark.parametrize("seed", range(6))
def test_p3_random_partitions(seed):
    rng = np.random.default_rng(100 + seed)
    C = int(rng.integers(1, 10))
    W = int(rng.integers(1, C + 1))
    cfg = Cfg(B=1, Hq=2, Hkv=1, D=4, C=C, W=W, seed=200 + seed)
    total = 40
    parts = []
    for _ in range(3):
        steps, t = [], 0
        while t < total:
            s = int(min(total - t, rng.integers(1, 2 * C + 2)))
            steps.append(s)
            t += s
        parts.append(steps)
    parts.append([1] * total)
    runs = [run_sequence(cfg, st, check=_check_layout(cfg)) for st in parts]
    for o, be in runs[1:]:
        for pos in range(total):
            assert np.array_equal(o[(0, pos)].view(np.uint8), runs[0][0][(0, pos)].view(np.uint8))
        L = oracle.resident_length(total, C, W)
        assert np.array_equal(be.K[:, :, :L], runs[0][1].K[:, :, :L])


# ---------------------------------------------------------------------------
# P4. Rollback: "Specify ... layout contract", Description: rejecting k drafts
# needs no cache edit and is exact iff L(T-k) == L(T) - k; Summary of Changes:
# verify 4 drafts, accept 2, resume from the untouched buffer and match the
# path that only ever appended the accepted tokens.
def test_p4_rollback_rule_both_directions():
    checked_exact = checked_inexact = 0
    for C, W in [(6, 4), (5, 5), (8, 3), (9, 6)]:
        cfg = Cfg(B=1, Hq=2, Hkv=1, D=4, C=C, W=W, seed=31, v_pos=True)
        for P in range(0, 3 * C):
            for S in range(1, C + 2):
                T = P + S
                for k in range(0, S):
                    exact = oracle.rollback_exact(T, k, C, W)
                    vers_a = Versions(1)
                    # path A: reach P, verify S drafts
                    _, be_a = run_sequence(cfg, ([P] if P else []) + [S], vers=vers_a)
                    # path B: reach P, append only the accepted S - k
                    vers_b = Versions(1)
                    steps_b = ([P] if P else []) + ([S - k] if S - k else [])
                    _, be_b = run_sequence(cfg, steps_b, vers=vers_b)
                    Lk = oracle.resident_length(T - k, C, W)
                    same = np.array_equal(be_a.V[:, :, :Lk], be_b.V[:, :, :Lk]) and \
                        np.array_equal(be_a.K[:, :, :Lk], be_b.K[:, :, :Lk])
                    assert same == exact, (C, W, P, S, k)
                    if exact:
                        checked_exact += 1
                        # resume both with the same next token (re-drawn)
                        syn = cfg.synth()
                        vers_a.bump(0, np.arange(T - k, T))
                        vers_b.bump(0, np.arange(T - k, T))
                        q, kk, vv = step_inputs(cfg, syn, np.array([T - k]), 1, vers_a)
                        _, oa, _ = be_a.step(1, [T - k], q, kk, vv)
                        _, ob, _ = be_b.step(1, [T - k], q, kk, vv)
                        assert np.array_equal(oa, ob)
                        L1 = oracle.resident_length(T - k + 1, C, W)
                        assert np.array_equal(be_a.V[:, :, :L1], be_b.V[:, :, :L1])
                    else:
                        checked_inexact += 1
                if P > 2 * C:
                    break
    assert checked_exact > 100 and checked_inexact > 50


def test_p4_tiny_contract_run_a_vs_b():
    """The tiny contract run: prefill 8 (S > C), 12 decodes, a 4-token verify
    step at P=20, reject k=2, one decode resumed at T=22 on the untouched
    buffer; versus the accepted-only path."""
    cfg = Cfg(B=1, Hq=4, Hkv=2, D=8, C=6, W=4, seed=1001, v_pos=True)
    assert oracle.rollback_exact(24, 2, 6, 4)
    syn = cfg.synth()
    va, vb = Versions(1), Versions(1)
    _, be_a = run_sequence(cfg, [8] + [1] * 12 + [4], vers=va)
    _, be_b = run_sequence(cfg, [8] + [1] * 12 + [2], vers=vb)
    va.bump(0, [22, 23])
    vb.bump(0, [22, 23])
    q, k, v = step_inputs(cfg, syn, np.array([22]), 1, va)
    _, oa, _ = be_a.step(1, [22], q, k, v)
    _, ob, _ = be_b.step(1, [22], q, k, v)
    assert np.array_equal(oa, ob)
    L = oracle.resident_length(23, 6, 4)
    assert np.array_equal(be_a.K[:, :, :L], be_b.K[:, :, :L])
    # and the inexact case P=19, S=4, k=2: L(21)=6 != L(23)-2=3
    assert oracle.resident_length(21, 6, 4) == 6 and oracle.resident_length(23, 6, 4) == 5
    assert not oracle.rollback_exact(23, 2, 6, 4)


# ---------------------------------------------------------------------------
# P6. Zero query: every visible score is equal, so each output is the mean of
# the visible V rows; with V[..., 0] = absolute position that mean is
# (lo + p) / 2 with lo = max(0, p - W + 1).
@pytest.mark.parametrize("C,W", [(6, 4), (7, 7), (9, 2)])
def test_p6_zero_query_closed_form(C, W):
    cfg = Cfg(B=1, Hq=4, Hkv=2, D=8, C=C, W=W, seed=61, v_pos=True, zero_q=True)
    outs, _ = run_sequence(cfg, [C + 2, 1, 3, 1, 2 * C + 1, 1])
    for (b, p), row in outs.items():
        lo = max(0, p - W + 1)
        got = row.reshape(cfg.Hq, cfg.D)[:, 0]
        assert np.all(got == np.float32((lo + p) / 2.0)), (p, got)


def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split("=", 1)
            vals[k.strip()] = np.array([float(x) for x in v.split()], dtype=np.float32)
    return vals


def _onehot_step(W):
    """Two cached positions and a two-token step; V rows one-hot at their
    position, K and Q zero (the printed example's inputs)."""
    D = 4
    p = oracle.make_params(1, 2, 1, 1, D, 6, W, 4, synth.F32)
    eye = np.eye(4, D, dtype=np.float32)
    past_k = np.zeros((1, 1, 6, D), np.float32)
    past_v = np.full((1, 1, 6, D), np.nan, np.float32)
    past_v[0, 0, :2] = eye[:2]
    q = np.zeros((1, 2, D), np.float32)
    k = np.zeros((1, 2, D), np.float32)
    v = eye[2:].reshape(1, 2, D).copy()
    st, out, _ = oracle.forward(p, q, k, v, past_k, past_v, np.array([3], np.int32))
    assert st == 0
    return out[0]


def test_p6_printed_causal_example():
    """"Fix CPU Attention causal mask for q_len=1 with past_key and
    kv_len > 1", Description / repro: the query at position 2 attends keys
    0, 1, 2 equally -> [1/3, 1/3, 1/3, 0]; the bug gave [0.25]*4."""
    g = _read_golden("p4_causal_onehot.txt")
    out = _onehot_step(W=4)
    assert np.array_equal(out[0], g["reference"])
    assert not np.array_equal(out[0], g["buggy"])
    assert np.array_equal(out[1], np.full(4, 0.25, np.float32))
    out2 = _onehot_step(W=2)  # window of two keys: positions 1 and 2
    assert np.array_equal(out2[0], np.array([0, 0.5, 0.5, 0], np.float32))


# ---------------------------------------------------------------------------
# P7. attention_bias in absolute key coordinates: "Specify ... layout
# contract", Description (last dimension stays total_sequence_length; the
# kernel selects the resident columns).
def test_p7_bias_spike_selects_absolute_column():
    cfg = Cfg(B=1, Hq=2, Hkv=1, D=4, C=6, W=5, seed=71, v_pos=True)
    syn = cfg.synth()
    vers = Versions(1)
    _, be = run_sequence(cfg, [13], vers=vers)   # T=13, L=5 rows: pos 8..12
    P, S = 13, 2
    total = P + S
    q, k, v = step_inputs(cfg, syn, np.array([P]), S, vers)
    for jstar in (10, 11, 13):
        bias = np.zeros((1, cfg.Hq, S, total), np.float32)
        bias[..., jstar] = 1000.0
        be2 = OracleBackend(cfg, be.K, be.V)
        st, out, _ = be2.step(S, [P + S - 1], q, k, v, bias=bias, total=total)
        assert st == 0
        vrow = as_f64(syn.kv_rows(synth.V, 0, 0, jstar, 0), cfg.dtype)
        for i in range(S):
            if jstar <= P + i and jstar > P + i - cfg.W:
                for h in range(cfg.Hq):
                    assert np.array_equal(out[0, i, h * 4:(h + 1) * 4].astype(np.float64), vrow)


def test_p7_bias_row_constant_and_weighted_mean():
    cfg = Cfg(B=1, Hq=2, Hkv=1, D=4, C=6, W=4, seed=72, v_pos=True, zero_q=True)
    syn = cfg.synth()
    vers = Versions(1)
    _, be = run_sequence(cfg, [9], vers=vers)
    P, S, total = 9, 3, 12
    q, k, v = step_inputs(cfg, syn, np.array([P]), S, vers)
    rng = np.random.default_rng(0)
    w = rng.uniform(0.5, 2.0, size=(cfg.Hq, S, total))
    bias = np.log(w).astype(np.float32)[None]
    st, out, _ = OracleBackend(cfg, be.K, be.V).step(S, [P + S - 1], q, k, v, bias=bias, total=total)
    for i in range(S):
        p = P + i
        js = np.arange(max(0, p - cfg.W + 1), p + 1)
        for h in range(cfg.Hq):
            ww = np.exp(bias[0, h, i, js].astype(np.float64))
            want = np.sum(ww * js) / np.sum(ww)      # V[...,0] = position
            assert abs(out[0, i, h * 4] - want) <= 2**-22 * abs(want)
    # a per-row constant leaves the output unchanged
    bias2 = bias + np.float32(3.0)
    _, out2, _ = OracleBackend(cfg, be.K, be.V).step(S, [P + S - 1], q, k, v, bias=bias2, total=total)
    assert np.allclose(out2, out, rtol=2**-21, atol=0)


def test_p7_bias_broadcast_dims():
    cfg = Cfg(B=2, Hq=2, Hkv=1, D=4, C=6, W=4, seed=73)
    syn = cfg.synth()
    vers = Versions(2)
    _, be = run_sequence(cfg, [7], vers=vers)
    P, S, total = 7, 2, 9
    q, k, v = step_inputs(cfg, syn, np.array([P, P]), S, vers)
    small = np.random.default_rng(1).normal(0, 0.1, (1, 1, S, total)).astype(np.float32)
    full = np.broadcast_to(small, (2, 2, S, total)).copy()
    _, o1, _ = OracleBackend(cfg, be.K, be.V).step(S, [8, 8], q, k, v, bias=small, total=total, bias_bcast=(0, 0))
    _, o2, _ = OracleBackend(cfg, be.K, be.V).step(S, [8, 8], q, k, v, bias=full, total=total)
    assert np.array_equal(o1, o2)


# ---------------------------------------------------------------------------
# P8. softcap (Investigation Report 1.3: logit soft-capping, 0 = disabled):
# zero query unchanged; saturation closed form; a huge cap equals none.
def test_p8_softcap_saturation_closed_form():
    D, c = 4, 1.5
    p = oracle.make_params(1, 1, 1, 1, D, 4, 4, 2, synth.F32, scale=1.0, softcap=c)
    past_k = np.zeros((1, 1, 4, D), np.float32)
    past_v = np.zeros((1, 1, 4, D), np.float32)
    past_k[0, 0, 0] = [1, 0, 0, 0]
    past_v[0, 0, 0] = [1, 0, 0, 0]
    q = np.array([[[100.0, 0, 0, 0]]], np.float32)
    k = np.array([[[-1.0, 0, 0, 0]]], np.float32)     # score -100 -> -c
    v = np.array([[[0, 1.0, 0, 0]]], np.float32)
    _, out, _ = oracle.forward(p, q, k, v, past_k, past_v, np.array([1], np.int32))
    e1, e2 = np.exp(c), np.exp(-c)
    want = np.array([e1 / (e1 + e2), e2 / (e1 + e2), 0, 0])
    assert np.all(np.abs(out[0, 0] - want) <= 2**-23 * np.abs(want) + 1e-30)


def test_p8_softcap_limits():
    base = Cfg(B=1, Hq=2, Hkv=1, D=8, C=6, W=4, seed=81)
    o_none, _ = run_sequence(base, [7, 1, 2])
    o_huge, _ = run_sequence(Cfg(**{**base.__dict__, "softcap": 1e30}), [7, 1, 2])
    for key in o_none:
        assert np.allclose(o_none[key], o_huge[key], rtol=2**-22, atol=0)
    o_small, _ = run_sequence(Cfg(**{**base.__dict__, "softcap": 0.05}), [7, 1, 2])
    assert any(not np.allclose(o_none[k], o_small[k], rtol=1e-3) for k in o_none)
    z = Cfg(**{**base.__dict__, "zero_q": True, "v_pos": True})
    o_z, _ = run_sequence(z, [7, 1])
    o_zc, _ = run_sequence(Cfg(**{**z.__dict__, "softcap": 0.7}), [7, 1])
    for key in o_z:
        assert np.array_equal(o_z[key], o_zc[key])


# ---------------------------------------------------------------------------
# P12. Softmax sink (Investigation Report 1.1 / 1.3 name head_sink, one value
# per query head, and smooth_softmax; reading: one more logit joins the
# denominator with a zero value row).  Zero query: all n visible scores are 0,
# so with V[..., 0] = absolute position each output is
# n (lo + p) / 2 / (n + e^sink); smooth_softmax alone is sink = 0.
@pytest.mark.parametrize("smooth,sink_std", [(True, 0.0), (False, 1.5), (True, 0.7)])
def test_p12_sink_zero_query_closed_form(smooth, sink_std):
    cfg = Cfg(B=1, Hq=4, Hkv=2, D=8, C=6, W=4, seed=121, v_pos=True, zero_q=True,
              smooth=smooth, sink_std=sink_std)
    sink = cfg.head_sink()
    sig = np.zeros(cfg.Hq) if sink is None else synth.from_storage(sink, cfg.dtype)
    outs, _ = run_sequence(cfg, [8, 1, 3, 1, 13, 1])
    for (b, p), row in outs.items():
        lo = max(0, p - cfg.W + 1)
        n = p - lo + 1
        want = n * (lo + p) / 2.0 / (n + np.exp(sig))
        got = row.reshape(cfg.Hq, cfg.D)[:, 0].astype(np.float64)
        assert np.all(np.abs(got - want) <= 2**-22 * np.abs(want) + 1e-30), (p, got, want)


def test_p12_sink_limits():
    base = Cfg(B=2, Hq=4, Hkv=2, D=8, C=7, W=5, seed=122)
    o_none, _ = run_sequence(base, [9, 1, 2, 4])
    # a sink logit far below every score changes nothing, bit for bit
    deep = Cfg(**{**base.__dict__, "sink_std": 1.0})
    sink = -1e30 * np.ones(base.Hq, np.float32)
    deep.head_sink = lambda: sink
    o_deep, _ = run_sequence(deep, [9, 1, 2, 4])
    for key in o_none:
        assert np.array_equal(o_none[key], o_deep[key])
    # a sink logit far above every score drives every output towards 0
    high = Cfg(**{**base.__dict__, "sink_std": 1.0})
    hsink = 60.0 * np.ones(base.Hq, np.float32)
    high.head_sink = lambda: hsink
    o_high, _ = run_sequence(high, [9, 1, 2, 4])
    for key in o_none:
        assert np.all(np.abs(o_high[key]) <= np.abs(o_none[key]).max() * 1e-20)
    # smooth_softmax is exactly a zero sink logit on every head
    o_smooth, _ = run_sequence(Cfg(**{**base.__dict__, "smooth": True}), [9, 1, 2, 4])
    zero = Cfg(**{**base.__dict__, "sink_std": 1.0})
    zsink = np.zeros(base.Hq, np.float32)
    zero.head_sink = lambda: zsink
    o_zero, _ = run_sequence(zero, [9, 1, 2, 4])
    for key in o_none:
        assert np.array_equal(o_smooth[key], o_zero[key])
        assert not np.array_equal(o_smooth[key], o_none[key])


# ---------------------------------------------------------------------------
# P9. GQA grouping (Investigation Report 1.3: num_heads Q heads share
# kv_num_heads K/V heads): with a zero query each Q head averages its KV
# head's V rows; MHA (Hq == Hkv) is the identity grouping.
@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (6, 3), (4, 4), (5, 1)])
def test_p9_grouping(Hq, Hkv):
    D, C, W = 4, 5, 3
    p = oracle.make_params(1, 2, Hq, Hkv, D, C, W, 7, synth.F32)
    past_k = np.zeros((1, Hkv, C, D), np.float32)
    past_v = np.zeros((1, Hkv, C, D), np.float32)
    for g in range(Hkv):
        past_v[0, g] = g + 1.0
    q = np.zeros((1, 2, Hq * D), np.float32)
    k = np.zeros((1, 2, Hkv * D), np.float32)
    v = np.repeat(np.arange(1, Hkv + 1, dtype=np.float32), D)[None, None, :].repeat(2, 1).copy()
    _, out, _ = oracle.forward(p, q, k, v, past_k, past_v, np.array([6], np.int32))
    for h in range(Hq):
        assert np.all(out[0, :, h * D:(h + 1) * D] == h // (Hq // Hkv) + 1.0)


# ---------------------------------------------------------------------------
# P10. Staging criterion: "[CPU] Add windowed kv cache for GQA", staging for
# hazardous steps.  Where the plan says "no hazard", compacting first and
# attending over the cache alone gives byte-identical outputs and caches;
# where it says "hazard", compacting first loses a key some query reads.
def test_p10_hazard_criterion_is_tight():
    n_h = n_ok = 0
    for C in range(1, 11):
        for W in range(1, C + 1):
            cfg = Cfg(B=1, Hq=2, Hkv=1, D=2, C=C, W=W, seed=C * 16 + W)
            syn = cfg.synth()
            vers = Versions(1)
            for P in range(0, 2 * C + 3):
                _, be = run_sequence(cfg, [P] if P else [], vers=vers)
                for S in range(1, 2 * C + 2):
                    q, k, v = step_inputs(cfg, syn, np.array([P]), S, vers)
                    p = cfg.params(S, P + S)
                    _, plan = oracle.plan(p, np.array([P + S - 1]))
                    hazard = plan[0, 7]
                    a = OracleBackend(cfg, be.K, be.V)
                    _, oa, _ = a.step(S, [P + S - 1], q, k, v)
                    bk, bv = be.K.copy(), be.V.copy()
                    st, ob = oracle.forward_compact_first(p, q, k, v, bk, bv,
                                                          np.array([P + S - 1], np.int32))
                    if hazard:
                        n_h += 1
                        assert st == 5, (C, W, P, S)
                    else:
                        n_ok += 1
                        assert st == 0, (C, W, P, S)
                        La = plan[0, 3]
                        assert np.array_equal(oa, ob)
                        assert np.array_equal(a.K[:, :, :La], bk[:, :, :La])
                        assert np.array_equal(a.V[:, :, :La], bv[:, :, :La])
    assert n_h > 100 and n_ok > 100


def test_p10_decode_never_hazardous():
    for C in range(1, 40):
        for W in range(1, C + 1):
            T = np.arange(1, 400)
            p = oracle.make_params(len(T), 1, 1, 1, 1, C, W, 400)
            st, plan = oracle.plan(p, T - 1)
            assert st == 0 and not plan[:, 7].any()


# ---------------------------------------------------------------------------
# P11. Printed facts of "[CPU] Add windowed kv cache for GQA": C = W + 8 with
# 400 decode steps gives about 44 compactions (Tests table); at C = W = 128
# every decode moves C - 1 rows, 0.50 MiB per token for 8 KV heads x 64 fp32
# (key design decisions); the C = 384 cache is 1.50 MiB (Performance).
def test_p11_printed_facts():
    W, C = 128, 136
    T = 512 + np.arange(1, 401)
    p = oracle.make_params(len(T), 1, 64, 8, 64, C, W, 2000)
    _, plan = oracle.plan(p, T - 1)
    events = int(np.count_nonzero(plan[:, 5] > 0))
    assert 44 <= events <= 45
    assert list(T[plan[:, 5] > 0][:3]) == [515, 524, 533]
    p = oracle.make_params(3, 1, 64, 8, 64, 128, 128, 2000)
    _, plan = oracle.plan(p, np.array([300, 700, 1500]))
    moved = plan[:, 4] * 8 * 2 * 64 * 4          # kept rows x heads x (K,V) x row
    assert np.all(plan[:, 4] == 127)
    assert round(moved[0] / 2**20, 2) == 0.50
    assert 8 * 2 * 384 * 64 * 4 / 2**20 == 1.5


def test_invalid_items_zero_output_untouched_cache():
    cfg = Cfg(B=3, Hq=2, Hkv=1, D=4, C=6, W=4, seed=91)
    syn = cfg.synth()
    vers = Versions(3)
    _, be = run_sequence(cfg, [5], vers=vers)
    q, k, v = step_inputs(cfg, syn, np.array([5, 5, 5]), 2, vers)
    before = be.snapshot()
    seq = np.array([6, 0, 6], np.int32)      # item 1: T=1 < S=2
    st, out, plan = be.step(2, seq, q, k, v, total=7)
    assert st == 4
    assert np.all(out[1] == 0) and np.all(plan[1] == -1)
    assert np.array_equal(be.K[1].view(np.uint8), before[0][1].view(np.uint8))
    seq = np.array([6, 6, 9], np.int32)      # item 2: T=10 > total=7
    st, out, plan = OracleBackend(cfg, *before).step(2, seq, q, k, v, total=7)
    assert st == 4 and np.all(out[2] == 0)


def test_argument_errors():
    p = oracle.make_params(1, 1, 3, 2, 4, 6, 4, 8)
    z = np.zeros(64, np.float32)
    assert oracle.forward(p, z, z, z, z, z, np.array([0], np.int32))[0] == 1
    p = oracle.make_params(1, 1, 2, 2, 4, 6, 7, 8)   # W > C
    assert oracle.forward(p, z, z, z, z, z, np.array([0], np.int32))[0] == 1
    p = oracle.make_params(1, 1, 2, 2, 4, 6, 0, 8)   # W < 1
    assert oracle.forward(p, z, z, z, z, z, np.array([0], np.int32))[0] == 1
    p = oracle.make_params(1, 1, 1, 1, 4, 2, 2, 8)
    big = np.zeros(16, np.float32)
    part = big[4:]                                   # partial overlap
    st = oracle.lib().swgqa_oracle_forward(
        p, z.ctypes.data, z.ctypes.data, z.ctypes.data, big.ctypes.data,
        big.ctypes.data, np.array([0], np.int32).ctypes.data, None, None, None, None, None,
        z.ctypes.data, part.ctypes.data, part.ctypes.data, None)
    assert st == 3
    p = oracle.make_params(1, 1, 2, 2, 4, 6, 4, 8, smooth_softmax=3)
    assert oracle.forward(p, z, z, z, z, z, np.array([0], np.int32))[0] == 1


# ---------------------------------------------------------------------------
# P13. Rotary embedding (Investigation Report 1.1 / 1.3 name cos_cache,
# sin_cache, position_ids, do_rotary and rotary_interleaved; reading: the pair
# (k, k + D/2) -- or (2k, 2k + 1) interleaved -- of a query or new key row at
# position pos is rotated by the angle whose cosine and sine are
# cos_cache[pos][k], sin_cache[pos][k]).  Observable through the stored keys
# (present rows are rotated keys) and the outputs.
def _rope_tables(rows, D, base=10000.0):
    k = np.arange(D // 2)
    ang = np.arange(rows)[:, None] * base ** (-2.0 * k[None, :] / D)
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def _rope_step(cfg, S, q, k, v, past_k, past_v, seq, cos, sin, interleaved=0, pos_ids=None,
               rows=None):
    p = oracle.make_params(cfg.B, S, cfg.Hq, cfg.Hkv, cfg.D, cfg.C, cfg.W, int(seq.max()) + 1,
                           cfg.dtype, do_rotary=1, rotary_interleaved=interleaved,
                           rotary_cache_rows=cos.shape[0] if rows is None else rows)
    K, V = past_k.copy(), past_v.copy()
    st, out, plan = oracle.forward(p, q, k, v, K, V, seq, cos_cache=cos, sin_cache=sin,
                                   position_ids=pos_ids)
    return st, out, K, V


def _rope_inputs(cfg, S, P):
    syn = cfg.synth()
    q, k, v = syn.step_inputs(np.array(P), S)
    K = np.zeros((cfg.B, cfg.Hkv, cfg.C, cfg.D), np.float32)
    V = np.zeros_like(K)
    return q, k, v, K, V


def test_p13_rotary_identity_table():
    cfg = Cfg(B=2, Hq=4, Hkv=2, D=8, C=12, W=6, seed=131)
    q, k, v, K, V = _rope_inputs(cfg, 9, [0, 0])
    seq = np.array([8, 8], np.int32)
    ones, zeros = np.ones((16, 4), np.float32), np.zeros((16, 4), np.float32)
    st, out, Kr, Vr = _rope_step(cfg, 9, q, k, v, K, V, seq, ones, zeros)
    p = cfg.params(9, 9)
    K0, V0 = K.copy(), V.copy()
    st0, out0, _ = oracle.forward(p, q, k, v, K0, V0, seq)
    assert st == 0 and st0 == 0
    assert np.array_equal(out, out0) and np.array_equal(Kr, K0) and np.array_equal(Vr, V0)


def test_p13_rotary_is_complex_rotation():
    """Stored keys equal (a + ib) e^{i angle}, computed by numpy's complex
    multiplication, to binary32 rounding; values are not rotated."""
    cfg = Cfg(B=1, Hq=2, Hkv=2, D=16, C=40, W=40, seed=132)
    S = 20
    q, k, v, K, V = _rope_inputs(cfg, S, [0])
    cos, sin = _rope_tables(64, cfg.D)
    st, _, Kr, Vr = _rope_step(cfg, S, q, k, v, K, V, np.array([S - 1], np.int32), cos, sin)
    assert st == 0
    kk = k.reshape(S, cfg.Hkv, cfg.D).astype(np.float64)
    z = (kk[..., :8] + 1j * kk[..., 8:]) * (cos[:S, None, :] + 1j * sin[:S, None, :]).astype(np.complex128)
    want = np.concatenate([z.real, z.imag], axis=-1)             # (S, Hkv, D)
    got = Kr[0, :, :S].transpose(1, 0, 2).astype(np.float64)
    assert np.all(np.abs(got - want) <= 4 * 2**-24 * (np.abs(kk).max(-1, keepdims=True) + 1e-30))
    assert np.array_equal(Vr[0, :, :S].transpose(1, 0, 2), v.reshape(S, cfg.Hkv, cfg.D))


def _decode_bits(a, dtype):
    """Element storage -> float32 values (exact for every element type)."""
    a = np.asarray(a)
    if dtype == synth.F32:
        return a.astype(np.float32)
    if dtype == synth.F16:
        return a.view(np.float16).astype(np.float32)
    return (a.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _round_bits(x32, dtype):
    """float32 values -> element storage, nearest-even: numpy's IEEE cast for
    fp16, torch's cast for bf16 (neither is the oracle's encoder)."""
    import torch
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == synth.F32:
        return x32
    if dtype == synth.F16:
        return x32.astype(np.float16).view(np.uint16)
    return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _rne_exact(x64, dtype):
    """Values rounded once, nearest-even, from float64 straight to the
    element type (no binary32 step): the alternative reading a pin must tell
    apart.  frexp / ldexp / rint arithmetic, written for this test only."""
    p, emin = {synth.F32: (24, -126), synth.F16: (11, -14), synth.BF16: (8, -126)}[dtype]
    ax = np.abs(x64)
    _, e = np.frexp(ax)
    q = np.maximum(e - 1, emin) - (p - 1)
    r = np.ldexp(np.rint(np.ldexp(ax, -q)), q)
    return _round_bits(np.where(x64 < 0, -r, r).astype(np.float32), dtype)


def _numpy_rotary(x, cos, sin, pos, dtype, interleaved, direct=False):
    """(B, S, H, D) storage rotated pair by pair: each product, the difference
    and the sum rounded to binary32 (numpy float32 ufuncs, one rounding per
    operation), the result to the element type.  direct=True instead forms
    each component exactly (float64 holds products of two binary32 values)
    and rounds it once to the element type -- a fused multiply-add for fp32,
    no binary32 step for fp16 / bf16."""
    xf = _decode_bits(x, dtype)
    c = _decode_bits(cos, dtype)[pos][:, :, None, :]
    s = _decode_bits(sin, dtype)[pos][:, :, None, :]
    half = xf.shape[-1] // 2
    ia = np.arange(0, 2 * half, 2) if interleaved else np.arange(half)
    ib = ia + 1 if interleaved else ia + half
    a, b = xf[..., ia], xf[..., ib]
    if direct:
        a64, b64, c64, s64 = (t.astype(np.float64) for t in (a, b, c, s))
        out = np.empty(xf.shape, np.float64)
        out[...] = xf
        out[..., ia] = a64 * c64 - b64 * s64
        out[..., ib] = b64 * c64 + a64 * s64
        return _rne_exact(out, dtype)
    ra = np.float32(a * c) - np.float32(b * s)
    rb = np.float32(b * c) + np.float32(a * s)
    out = xf.copy()
    out[..., ia] = ra
    out[..., ib] = rb
    return _round_bits(out, dtype)


def _hard_fp16_rotations(n_want=24, seed=1361):
    """fp16 quadruples (a, b, c, s) where one rotated component rounds
    differently through binary32 than straight from the exact value (about 2
    in 10^5 random draws; products of fp16 values are exact in binary32, so
    only the sum or difference is rounded there)."""
    rng = np.random.default_rng(seed)
    found = []
    while len(found) < n_want:
        n = 1 << 20
        ab = synth.to_storage(rng.normal(size=(n, 2)).astype(np.float32), synth.F16)
        ang = rng.uniform(0.0, 100.0, size=n)
        c = synth.to_storage(np.cos(ang), synth.F16)
        s = synth.to_storage(np.sin(ang), synth.F16)
        x = ab.reshape(1, n, 1, 2)
        pos = np.arange(n)[None, :]
        per = _numpy_rotary(x, c[:, None], s[:, None], pos, synth.F16, 0)
        alt = _numpy_rotary(x, c[:, None], s[:, None], pos, synth.F16, 0, direct=True)
        hit = np.nonzero((per != alt).any(-1)[0, :, 0])[0]
        found += [(ab[i, 0], ab[i, 1], c[i], s[i]) for i in hit]
    return np.array(found[:n_want], dtype=np.uint16)


def _check_rotary_step(cfg, S, q, k, v, K, V, seq, cos, sin, pos, interleaved):
    """One prefill step through the oracle with rotary: stored keys and (via
    an un-rotated step fed the rotated rows) outputs against numpy's per-
    operation binary32 rotation.  Returns numpy's rotated keys."""
    dtype = cfg.dtype
    explicit = pos if not np.array_equal(pos, np.broadcast_to(np.arange(S), pos.shape)) else None
    st, out, Kr, Vr = _rope_step(cfg, S, q, k, v, K, V, seq, cos, sin,
                                 interleaved=interleaved, pos_ids=explicit)
    assert st == 0
    k4 = k.reshape(cfg.B, S, cfg.Hkv, cfg.D)
    want_k = _numpy_rotary(k4, cos, sin, pos, dtype, interleaved)
    got_k = np.ascontiguousarray(Kr[:, :, :S].transpose(0, 2, 1, 3))
    assert np.array_equal(got_k.view(np.uint8), want_k.view(np.uint8))
    assert np.array_equal(Vr[:, :, :S].transpose(0, 2, 1, 3), v.reshape(k4.shape))
    q4 = q.reshape(cfg.B, S, cfg.Hq, cfg.D)
    want_q = _numpy_rotary(q4, cos, sin, pos, dtype, interleaved)
    K0, V0 = K.copy(), V.copy()
    st0, out0, _ = oracle.forward(cfg.params(S, S), want_q.reshape(q.shape),
                                  want_k.reshape(k.shape), v, K0, V0, seq)
    assert st0 == 0 and np.array_equal(out.view(np.uint8), out0.view(np.uint8))
    return k4, want_k


@pytest.mark.parametrize("interleaved", [0, 1])
@pytest.mark.parametrize("dtype", [synth.F32, synth.F16, synth.BF16])
def test_p13_rotary_rounding_is_binary32_per_operation(dtype, interleaved):
    """Stored keys equal, bit for bit, numpy's float32 evaluation of
    (a c - b s, b c + a s) one operation at a time, rounded to the element
    type; the query rotation likewise (an un-rotated step fed numpy's rotated
    rows returns bit-identical outputs).  Default and explicit (left-padded)
    positions.  Discrimination on these inputs: for fp32 a fused multiply-add
    (exact component, one rounding) differs; for fp16 rounding the exact
    component straight to fp16 differs on searched inputs; for bf16 no input
    separates the two (products of 8-bit significands and their sums stay
    exact in binary32 or round away from bf16 midpoints), so the per-
    operation result must equal the exact component rounded once."""
    cfg = Cfg(B=2, Hq=4, Hkv=2, D=64, C=300, W=300, seed=136, dtype=dtype)
    S = 160
    q, k, v, K, V = _rope_inputs(cfg, S, [0, 0])
    if dtype != synth.F32:
        K, V = K.astype(np.uint16), V.astype(np.uint16)
    cos, sin = synth.rotary_tables(512, cfg.D, dtype, base=50.0)
    seq = np.array([S - 1, S - 1], np.int32)
    told_apart = False
    for pos in (np.stack([np.arange(S), np.arange(S)]),
                np.stack([np.arange(S) + 3, np.arange(S) + 211])):
        k4, want_k = _check_rotary_step(cfg, S, q, k, v, K, V, seq, cos, sin, pos, interleaved)
        alt = _numpy_rotary(k4, cos, sin, pos, dtype, interleaved, direct=True)
        if dtype == synth.BF16:
            assert np.array_equal(alt, want_k)
        told_apart |= not np.array_equal(alt, want_k)
    if dtype == synth.F16:
        # searched inputs: pair 0 of new key row i and table row i
        hard = _hard_fp16_rotations()
        n = len(hard)
        hc = Cfg(B=1, Hq=1, Hkv=1, D=8, C=n, W=n, seed=137, dtype=dtype)
        q, k, v, K, V = _rope_inputs(hc, n, [0])
        K, V = K.astype(np.uint16), V.astype(np.uint16)
        k = k.reshape(1, n, 8).copy()
        ia, ib = (0, 1) if interleaved else (0, 4)
        k[0, :, ia], k[0, :, ib] = hard[:, 0], hard[:, 1]
        hcos, hsin = synth.rotary_tables(n, 8, dtype)
        hcos, hsin = hcos.copy(), hsin.copy()
        hcos[:, 0], hsin[:, 0] = hard[:, 2], hard[:, 3]
        pos = np.arange(n)[None, :]
        k4, want_k = _check_rotary_step(hc, n, q, k.reshape(1, n * 1 * 8), v, K, V,
                                        np.array([n - 1], np.int32), hcos, hsin, pos, interleaved)
        alt = _numpy_rotary(k4, hcos, hsin, pos, dtype, interleaved, direct=True)
        told_apart |= not np.array_equal(alt, want_k)
    assert told_apart or dtype == synth.BF16, "these inputs cannot tell the readings apart"


def test_p13_interleaved_is_a_permutation_of_halves():
    """Interleaved pairs (2k, 2k+1) on a row equal half pairs (k, k + D/2) on
    the row with its even elements first and odd elements second."""
    cfg = Cfg(B=1, Hq=2, Hkv=1, D=8, C=10, W=10, seed=133)
    S = 7
    q, k, v, K, V = _rope_inputs(cfg, S, [0])
    cos, sin = _rope_tables(16, cfg.D)
    seq = np.array([S - 1], np.int32)
    perm = np.concatenate([np.arange(0, 8, 2), np.arange(1, 8, 2)])
    _, _, Ki, _ = _rope_step(cfg, S, q, k, v, K, V, seq, cos, sin, interleaved=1)
    kp = np.ascontiguousarray(k.reshape(1, S, 1, 8)[..., perm].reshape(k.shape))
    qp = np.ascontiguousarray(q.reshape(1, S, 2, 8)[..., perm].reshape(q.shape))
    _, _, Kh, _ = _rope_step(cfg, S, qp, kp, v, K, V, seq, cos, sin, interleaved=0)
    assert np.array_equal(Ki[0, 0, :S][:, perm], Kh[0, 0, :S])


def test_p13_relative_positions_and_position_ids():
    """All keys rotated in one prefill step: shifting every position by a
    constant through position_ids leaves every score, hence every output,
    unchanged (to rounding); explicit positions P + i equal the default."""
    cfg = Cfg(B=1, Hq=4, Hkv=2, D=16, C=30, W=9, seed=134)
    S = 24
    q, k, v, K, V = _rope_inputs(cfg, S, [0])
    cos, sin = _rope_tables(128, cfg.D)
    seq = np.array([S - 1], np.int32)
    st, base, Kb, _ = _rope_step(cfg, S, q, k, v, K, V, seq, cos, sin)
    st2, same, Ks, _ = _rope_step(cfg, S, q, k, v, K, V, seq, cos, sin,
                                  pos_ids=np.arange(S)[None, :])
    assert st == 0 and st2 == 0 and np.array_equal(base, same) and np.array_equal(Kb, Ks)
    st3, shifted, _, _ = _rope_step(cfg, S, q, k, v, K, V, seq, cos, sin,
                                    pos_ids=np.arange(S)[None, :] + 37)
    assert st3 == 0
    assert np.allclose(shifted, base, rtol=2e-4, atol=2e-5)
    assert not np.allclose(shifted, _rope_step(cfg, S, q, k, v, K, V, seq, np.ones_like(cos),
                                               np.zeros_like(sin))[1], rtol=1e-3)


def test_p13_position_outside_the_tables_is_an_item_error():
    cfg = Cfg(B=2, Hq=2, Hkv=1, D=8, C=10, W=4, seed=135)
    q, k, v, K, V = _rope_inputs(cfg, 3, [0, 0])
    cos, sin = _rope_tables(8, cfg.D)
    seq = np.array([2, 2], np.int32)
    pos = np.array([[0, 1, 2], [6, 7, 8]])          # item 1 reaches row 8 of 8
    st, out, Kr, _ = _rope_step(cfg, 3, q, k, v, K, V, seq, cos, sin, pos_ids=pos)
    assert st == 4 and np.all(out[1] == 0) and np.all(Kr[1] == 0) and not np.all(Kr[0] == 0)


# ---------------------------------------------------------------------------
# P14. Quantized cache (Investigation Report 1.1 names the inputs k_scale /
# v_scale, "KV cache quantization scale", and a cache type T_CACHE apart from
# T; reading: int8 codes, one scale per tensor, a cache element stands for
# code * scale, a new element x is stored as the binary32 quotient x / scale
# rounded to an integer with ties to even and saturated to [-128, 127]; the
# step attends to every row in that dequantized form, new rows included).
def _q_forward(cfg, S, q, k, v, K8, V8, seq, ks, vs, total=None):
    total = int(np.max(seq)) + 1 if total is None else total
    p = oracle.make_params(len(seq), S, cfg.Hq, cfg.Hkv, cfg.D, cfg.C, cfg.W, total, cfg.dtype,
                           cfg.scale, cfg.softcap, kv_cache_type=1, k_scale=ks, v_scale=vs)
    K, V = K8.copy(), V8.copy()
    st, out, plan = oracle.forward(p, q, k, v, K, V, np.asarray(seq, np.int32))
    return st, out, K, V


def _grid_rows(rng, shape, step, dtype):
    """Elements code * step for random codes in [-128, 127]: exact in every
    element type (at most 8 significant bits)."""
    codes = rng.integers(-128, 128, size=shape)
    return codes.astype(np.int8), synth.to_storage((codes * step).astype(np.float32), dtype)


@pytest.mark.parametrize("dtype", [synth.F32, synth.F16, synth.BF16])
def test_p14_grid_values_equal_the_plain_cache(dtype):
    """New rows whose elements are code * scale exactly: the stored codes are
    those codes, and every output equals the plain cache's bit for bit (the
    dequantized rows are the original values), across a staged prefill and
    decode steps that read int8 resident rows."""
    cfg = Cfg(B=2, Hq=4, Hkv=2, D=8, C=10, W=6, dtype=dtype, seed=141)
    rng = np.random.default_rng(141)
    ks, vs = 2.0 ** -3, 2.0 ** -5
    syn = cfg.synth()
    K8 = np.zeros((2, cfg.Hkv, cfg.C, cfg.D), np.int8)
    V8 = np.zeros_like(K8)
    Kp = scenario_nan((2, cfg.Hkv, cfg.C, cfg.D), dtype)
    Vp = scenario_nan((2, cfg.Hkv, cfg.C, cfg.D), dtype)
    T = np.zeros(2, np.int64)
    for S in [7, 1, 1, 3, 1, 12, 1]:
        q, _, _ = syn.step_inputs(T, S)
        kc, k = _grid_rows(rng, (2, S, cfg.Hkv * cfg.D), ks, dtype)
        vc, v = _grid_rows(rng, (2, S, cfg.Hkv * cfg.D), vs, dtype)
        seq = (T + S - 1).astype(np.int32)
        st, out, K8, V8 = _q_forward(cfg, S, q, k, v, K8, V8, seq, ks, vs)
        p = oracle.make_params(2, S, cfg.Hq, cfg.Hkv, cfg.D, cfg.C, cfg.W, int(seq.max()) + 1, dtype)
        st0, out0, plan = oracle.forward(p, q, k, v, Kp, Vp, seq)
        assert st == 0 and st0 == 0
        assert np.array_equal(np.asarray(out).view(np.uint8), np.asarray(out0).view(np.uint8))
        for b in range(2):
            La = int(plan[b, 3])
            assert np.array_equal(as_f64(Kp[b, :, :La], dtype), K8[b, :, :La] * ks)
            assert np.array_equal(as_f64(Vp[b, :, :La], dtype), V8[b, :, :La] * vs)
            # the newest rows are this step's codes
            n = min(S, La)
            got = K8[b, :, La - n:La]                               # (Hkv, n, D)
            want = kc[b, S - n:].reshape(n, cfg.Hkv, cfg.D).transpose(1, 0, 2)
            assert np.array_equal(got, want)
        T = T + S


def scenario_nan(shape, dtype):
    from tests.scenario import nan_array
    return nan_array(shape, dtype)


def test_p14_rounding_ties_to_even_and_saturation():
    cfg = Cfg(B=1, Hq=2, Hkv=1, D=16, C=4, W=4, seed=142)
    ks, vs = 0.25, 0.5
    mult = np.array([2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 1.5, -1.5,
                     1000.0, -1000.0, 127.5, -128.5, 126.5, -127.5, 0.0, 7.0])
    want = np.array([2, 4, -2, -4, 0, 0, 2, -2, 127, -128, 127, -128, 126, -128, 0, 7], np.int8)
    k = (mult * ks).astype(np.float32).reshape(1, 1, 16)
    v = (mult * vs).astype(np.float32).reshape(1, 1, 16)
    q = np.zeros((1, 1, 2 * 16), np.float32)
    K8 = np.zeros((1, 1, 4, 16), np.int8)
    st, _, K, V = _q_forward(cfg, 1, q, k, v, K8, K8.copy(), [0], ks, vs)
    assert st == 0
    assert np.array_equal(K[0, 0, 0], want) and np.array_equal(V[0, 0, 0], want)


def test_p14_scales_multiply_the_codes():
    """Doubling k_scale while halving the query, or doubling v_scale, moves
    every score / output by exactly that power of two: the key scale
    multiplies the key codes in the scores, the value scale the values."""
    cfg = Cfg(B=1, Hq=4, Hkv=2, D=8, C=12, W=9, seed=143)
    rng = np.random.default_rng(143)
    K8 = rng.integers(-128, 128, size=(1, 2, 12, 8)).astype(np.int8)
    V8 = rng.integers(-128, 128, size=(1, 2, 12, 8)).astype(np.int8)
    q = rng.normal(size=(1, 1, 32)).astype(np.float32)
    zero_kv = np.zeros((1, 1, 16), np.float32)       # the new row: code 0 at any scale
    seq = [10]                                       # P = 10 resident rows
    st, base, _, _ = _q_forward(cfg, 1, q, zero_kv, zero_kv, K8, V8, seq, 0.03, 0.07)
    st2, same, _, _ = _q_forward(cfg, 1, q * 0.5, zero_kv, zero_kv, K8, V8, seq, 0.06, 0.07)
    st3, dbl, _, _ = _q_forward(cfg, 1, q, zero_kv, zero_kv, K8, V8, seq, 0.03, 0.14)
    assert st == st2 == st3 == 0
    assert np.array_equal(base, same)
    assert np.array_equal(dbl, base * 2)
    st4, other, _, _ = _q_forward(cfg, 1, q, zero_kv, zero_kv, K8, V8, seq, 0.09, 0.07)
    assert not np.allclose(other, base)                # the key scale does enter


def test_p14_dequantized_rows_within_half_a_step():
    """Random elements inside the code range come back within scale / 2."""
    cfg = Cfg(B=1, Hq=2, Hkv=2, D=32, C=40, W=40, seed=144)
    syn = cfg.synth()
    ks, vs = 0.02, 0.03
    q, k, v = syn.step_inputs(np.array([0]), 30)
    K8 = np.zeros((1, 2, 40, 32), np.int8)
    st, _, K, V = _q_forward(cfg, 30, q, k, v, K8, K8.copy(), [29], ks, vs)
    assert st == 0
    kk = k.reshape(30, 2, 32).transpose(1, 0, 2).astype(np.float64)
    vv = v.reshape(30, 2, 32).transpose(1, 0, 2).astype(np.float64)
    for x, c, sc in [(kk, K[0, :, :30], ks), (vv, V[0, :, :30], vs)]:
        inside = np.abs(x) < 127 * sc
        assert inside.mean() > 0.9
        assert np.all(np.abs(c * sc - x)[inside] <= sc / 2 * (1 + 1e-6))


def test_p14_step_split_invariance():
    """Quantization is per element: an 8-token prefill plus a 4-token step
    and twelve 1-token steps leave the same codes and give the same outputs."""
    cfg = Cfg(B=1, Hq=4, Hkv=2, D=8, C=10, W=6, seed=145)
    syn = cfg.synth()
    ks, vs = 0.05, 0.04
    q, k, v = syn.step_inputs(np.array([0]), 12)
    K8 = np.zeros((1, 2, 10, 8), np.int8)

    def run(parts):
        K, V = K8.copy(), K8.copy()
        outs, t = [], 0
        for S in parts:
            sl = slice(t, t + S)
            st, out, K, V = _q_forward(cfg, S, np.ascontiguousarray(q[:, sl]),
                                       np.ascontiguousarray(k[:, sl]),
                                       np.ascontiguousarray(v[:, sl]), K, V, [t + S - 1], ks, vs)
            assert st == 0
            outs.append(out)
            t += S
        return np.concatenate(outs, axis=1), K, V

    oa, Ka, Va = run([8, 4])
    ob, Kb, Vb = run([1] * 12)
    L = oracle.resident_length(12, 10, 6)
    assert np.array_equal(oa, ob)
    assert np.array_equal(Ka[:, :, :L], Kb[:, :, :L]) and np.array_equal(Va[:, :, :L], Vb[:, :, :L])


def test_p14_zero_query_mean_of_dequantized_positions():
    """Zero query, V element 0 = absolute position, v_scale 1 (positions
    below 128 are exact codes): output element 0 is the window mean
    (lo + p) / 2."""
    cfg = Cfg(B=1, Hq=4, Hkv=2, D=8, C=9, W=5, seed=146, v_pos=True, zero_q=True)
    syn = cfg.synth()
    K8 = np.zeros((1, 2, 9, 8), np.int8)
    V8 = np.zeros_like(K8)
    T = 0
    for S in [6, 1, 1, 1, 4, 1, 1]:
        q, k, v = syn.step_inputs(np.array([T]), S)
        st, out, K8, V8 = _q_forward(cfg, S, q, k, v, K8, V8, [T + S - 1], 0.5, 1.0)
        assert st == 0
        o = out.reshape(S, 4, 8)[:, :, 0]
        for i in range(S):
            p = T + i
            lo = max(0, p - cfg.W + 1)
            assert np.allclose(o[i], (lo + p) / 2.0, rtol=0, atol=1e-6)
        T += S


def test_p14_argument_checks():
    cfg = Cfg(B=1, Hq=2, Hkv=1, D=8, C=4, W=4, seed=147)
    q = np.zeros((1, 1, 16), np.float32)
    k = np.zeros((1, 1, 8), np.float32)
    K8 = np.zeros((1, 1, 4, 8), np.int8)
    assert _q_forward(cfg, 1, q, k, k, K8, K8, [0], 0.0, 1.0)[0] == 1
    assert _q_forward(cfg, 1, q, k, k, K8, K8, [0], 1.0, float("inf"))[0] == 1
    p = oracle.make_params(1, 1, 2, 1, 8, 4, 4, 1, kv_cache_type=3, k_scale=1.0, v_scale=1.0)
    assert oracle.forward(p, q, k, k, K8.copy(), K8.copy(), np.zeros(1, np.int32))[0] == 2


# ---------------------------------------------------------------------------
# P15. fp8 E4M3 cache codes (kv_cache_type 2; the same reading as P14 with
# OCP E4M3 "FN" codes: nearest value, ties to the even code, magnitudes of 448
# or more saturated to 448, NaN to 0x7F, results of zero coded +0).
def test_p15_e4m3_values_equal_torch_float8():
    """Every one of the 256 codes decodes to torch's float8_e4m3fn value (an
    independent implementation of the OCP format), and the printed facts of
    the format hold: 448 largest, 2^-6 smallest normal, 2^-9 smallest
    subnormal, 0x7F / 0xFF NaN."""
    torch = pytest.importorskip("torch")
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = np.array([oracle.decode_e4m3(c) for c in range(256)])
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(ours[~np.isnan(ours)], ref[~np.isnan(ref)])
    assert oracle.decode_e4m3(0x7E) == 448.0 and oracle.decode_e4m3(0x08) == 2.0 ** -6
    assert oracle.decode_e4m3(0x01) == 2.0 ** -9 and np.isnan(oracle.decode_e4m3(0x7F))
    assert np.isnan(ours).sum() == 2


def test_p15_e4m3_rounding_against_torch():
    """Inside the range the code equals torch's float8 cast (nearest, ties to
    even) for random values, all midpoints between neighbouring codes and
    the codes themselves; saturation and +0 for results of zero are the
    reading's own (torch gives NaN and -0 there)."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(151)
    vals = np.concatenate([
        rng.normal(0, 30, 3000), rng.normal(0, 0.01, 1000),
        np.exp(rng.uniform(-12, 6, 1000)) * rng.choice([-1, 1], 1000)])
    table = np.array([oracle.decode_e4m3(c) for c in range(0x7F)])      # 0 .. 448
    mids = (table[1:] + table[:-1]) / 2
    vals = np.concatenate([vals, table, mids, -mids]).astype(np.float32)
    vals = vals[np.abs(vals) < 448]
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(int)
    ours = np.array([oracle.quantize_e4m3(float(v), 1.0) for v in vals])
    ref = np.where(ref == 0x80, 0, ref)                                   # -0 -> +0
    assert np.array_equal(ours, ref)
    assert oracle.quantize_e4m3(1000.0, 1.0) == 0x7E and oracle.quantize_e4m3(-1e30, 1.0) == 0xFE
    assert oracle.quantize_e4m3(float("nan"), 1.0) == 0x7F
    assert oracle.quantize_e4m3(-2.0 ** -11, 1.0) == 0


def test_p15_fp8_grid_values_equal_the_plain_cache():
    """New elements that are E4M3 values times the scale: the stored codes
    decode to them and the outputs equal the plain cache's bit for bit."""
    cfg = Cfg(B=2, Hq=4, Hkv=2, D=8, C=10, W=6, dtype=synth.F32, seed=152)
    rng = np.random.default_rng(152)
    ks, vs = 2.0 ** -4, 2.0 ** -3
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    vals = np.array([oracle.decode_e4m3(int(c)) for c in finite])
    syn = cfg.synth()
    K8 = np.zeros((2, cfg.Hkv, cfg.C, cfg.D), np.uint8)
    V8 = np.zeros_like(K8)
    Kp = scenario_nan((2, cfg.Hkv, cfg.C, cfg.D), cfg.dtype)
    Vp = scenario_nan((2, cfg.Hkv, cfg.C, cfg.D), cfg.dtype)
    T = np.zeros(2, np.int64)
    for S in [7, 1, 3, 1, 12, 1]:
        q, _, _ = syn.step_inputs(T, S)
        k = (rng.choice(vals, size=(2, S, cfg.Hkv * cfg.D)) * ks).astype(np.float32)
        v = (rng.choice(vals, size=(2, S, cfg.Hkv * cfg.D)) * vs).astype(np.float32)
        seq = (T + S - 1).astype(np.int32)
        p8 = oracle.make_params(2, S, cfg.Hq, cfg.Hkv, cfg.D, cfg.C, cfg.W, int(seq.max()) + 1,
                                cfg.dtype, kv_cache_type=2, k_scale=ks, v_scale=vs)
        st, out, _ = oracle.forward(p8, q, k, v, K8, V8, seq)
        p = oracle.make_params(2, S, cfg.Hq, cfg.Hkv, cfg.D, cfg.C, cfg.W, int(seq.max()) + 1, cfg.dtype)
        st0, out0, plan = oracle.forward(p, q, k, v, Kp, Vp, seq)
        assert st == 0 and st0 == 0
        assert np.array_equal(out.view(np.uint8), out0.view(np.uint8))
        dec = np.vectorize(oracle.decode_e4m3)
        for b in range(2):
            La = int(plan[b, 3])
            assert np.array_equal(dec(K8[b, :, :La]) * ks, Kp[b, :, :La].astype(np.float64))
            assert np.array_equal(dec(V8[b, :, :La]) * vs, Vp[b, :, :La].astype(np.float64))
        T = T + S


def test_p15_fp8_relative_error_and_saturation():
    """Normal-range elements come back within 2^-4 relative (half a step of
    the 3-bit mantissa); far values saturate to +-448 * scale."""
    cfg = Cfg(B=1, Hq=2, Hkv=2, D=32, C=40, W=40, seed=153)
    syn = cfg.synth()
    q, k, v = syn.step_inputs(np.array([0]), 30)
    k[0, 0, :4] = [1e6, -1e6, 5e3, -5e3]
    p = oracle.make_params(1, 30, 2, 2, 32, 40, 40, 30, kv_cache_type=2, k_scale=0.01, v_scale=0.02)
    K8 = np.zeros((1, 2, 40, 32), np.uint8)
    V8 = np.zeros_like(K8)
    st, _, _ = oracle.forward(p, q, k, v, K8, V8, np.array([29], np.int32))
    assert st == 0
    assert list(K8[0, 0, 0, :4]) == [0x7E, 0xFE, 0x7E, 0xFE]
    dec = np.vectorize(oracle.decode_e4m3)
    vv = v.reshape(30, 2, 32).transpose(1, 0, 2).astype(np.float64)
    got = dec(V8[0, :, :30]) * 0.02
    normal = np.abs(vv) >= 2.0 ** -6 * 0.02
    assert np.all(np.abs(got - vv)[normal] <= 2.0 ** -4 * np.abs(vv)[normal] * (1 + 1e-9))
