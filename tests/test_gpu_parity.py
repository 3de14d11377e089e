"""GPU parity: libswgqa (HIP, through the C ABI) against the CPU oracle.

Outputs within 1e-5 (fp32) / 2e-3 (fp16, bf16) of max(1, |oracle|); present
rows [0, L(T)) and plan records bit-exact; unspecified rows NaN-poisoned
before every step; canaries around every cache buffer; both buffer modes
(shared past == present, and separate buffers).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from tests.parity import Lockstep, say
from tests.scenario import Cfg, Versions, seeded_cache, step_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sliding_window_gqa_02_amd as sw
    sw.load()


# ---------------------------------------------------------------------------
def test_plan_kernel_matches_oracle():
    import sliding_window_gqa_02_amd as sw
    from tests.gpu_backend import to_dev
    rng = np.random.default_rng(5)
    for C, W, S in [(6, 4, 1), (6, 4, 8), (384, 128, 1), (136, 128, 1), (1032, 1024, 32),
                    (1055, 1024, 8), (4608, 4096, 1), (1, 1, 3), (9, 9, 20)]:
        seq = np.concatenate([rng.integers(-3, 40_000, size=200), [S - 1, S - 2, 2**31 - 2]])
        seq = seq.astype(np.int32)
        total = 39_000
        p = sw.make_params(len(seq), S, 2, 1, 8, C, W, total)
        out = torch.zeros((len(seq), 8), dtype=torch.int64, device="cuda:0")
        sw.plan(p, to_dev(seq), out)
        torch.cuda.synchronize()
        po = oracle.make_params(len(seq), S, 2, 1, 8, C, W, total)
        _, ref = oracle.plan(po, seq)
        assert np.array_equal(out.cpu().numpy(), ref), (C, W, S)


# ---------------------------------------------------------------------------
# The tiny contract check: B=1, Hq=4, Hkv=2, D=8, fp32, W=4, C=6, V[...,0] =
# absolute position; 8-token prefill (S > C: staged), 12 decodes, a 4-token
# verify step at P=20 with k=2 rejected, one decode resumed at T=22 on the
# untouched buffer (run A) vs the accepted-only path (run B); the same
# 4 tokens as one step vs four 1-token steps (run C); zero query (run D).
TINY = Cfg(B=1, Hq=4, Hkv=2, D=8, C=6, W=4, seed=1001, v_pos=True)


@pytest.mark.parametrize("mode", ["shared", "separate"])
def test_tiny_contract_runs(mode):
    say(f"tiny contract, mode={mode}")
    # run A
    A = Lockstep(TINY, mode=mode)
    A.step([0], 8)
    for T in range(9, 21):
        A.step([T - 1], 1)
    A.step([20], 4)                      # verify 4 drafts
    assert oracle.rollback_exact(24, 2, TINY.C, TINY.W)
    A.vers.bump(0, [22, 23])             # k=2 rejected: positions 22, 23 re-drawn
    outA, _, _ = A.step([22], 1)         # resume at T=22 -> 23, buffer untouched
    # run B: accepted tokens only
    B = Lockstep(TINY, mode=mode)
    B.step([0], 8)
    for T in range(9, 21):
        B.step([T - 1], 1)
    B.step([20], 2)
    B.vers.bump(0, [22, 23])
    outB, _, _ = B.step([22], 1)
    assert np.array_equal(outA, outB)
    L = oracle.resident_length(23, TINY.C, TINY.W)
    ka, _ = A.gpu.present_host()
    kb, _ = B.gpu.present_host()
    assert np.array_equal(ka[:, :, :L], kb[:, :, :L])
    # run C: one 4-token step vs four single steps after the 8-token prefill
    C1 = Lockstep(TINY, mode=mode)
    C1.step([0], 8)
    o4, _, _ = C1.step([8], 4)
    C4 = Lockstep(TINY, mode=mode)
    C4.step([0], 8)
    singles = [C4.step([8 + i], 1)[0] for i in range(4)]
    # presents are byte-identical; outputs come from differently shaped query
    # tiles (other summation orders), so they agree to the fp32 tolerance
    for i in range(4):
        assert np.allclose(o4[:, i], singles[i][:, 0], rtol=1e-5, atol=1e-5)
    L = oracle.resident_length(12, TINY.C, TINY.W)
    k1, v1 = C1.gpu.present_host()
    k4, v4 = C4.gpu.present_host()
    assert np.array_equal(k1[:, :, :L], k4[:, :, :L]) and np.array_equal(v1[:, :, :L], v4[:, :, :L])
    # run D: zero query -> mean of the visible V rows, element 0 = (lo + p) / 2
    zq = Cfg(**{**TINY.__dict__, "zero_q": True})
    Dz = Lockstep(zq, mode=mode)
    outs = [Dz.step([0], 8)[0]] + [Dz.step([T - 1], 1)[0] for T in range(9, 15)]
    pos = list(range(8)) + list(range(8, 14))
    rows = np.concatenate([o[0] for o in outs], axis=0)
    for p, r in zip(pos, rows):
        lo = max(0, p - TINY.W + 1)
        assert np.allclose(r.reshape(4, 8)[:, 0], (lo + p) / 2.0, rtol=1e-6)


# ---------------------------------------------------------------------------
SMALL = [
    Cfg(B=2, Hq=2, Hkv=2, D=8, C=5, W=5, seed=11),
    Cfg(B=1, Hq=3, Hkv=1, D=16, C=7, W=1, seed=12),
    Cfg(B=2, Hq=4, Hkv=1, D=8, C=9, W=3, seed=13, dtype=synth.F16),
    Cfg(B=1, Hq=2, Hkv=1, D=32, C=8, W=6, seed=14, dtype=synth.BF16, softcap=2.0),
    Cfg(B=3, Hq=8, Hkv=2, D=64, C=40, W=33, seed=16),
    Cfg(B=2, Hq=16, Hkv=2, D=128, C=70, W=64, seed=17, dtype=synth.BF16, softcap=30.0),
    Cfg(B=1, Hq=4, Hkv=4, D=256, C=20, W=17, seed=18, dtype=synth.F16),
]


@pytest.mark.parametrize("mode", ["shared", "separate"])
@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: f"C{c.C}W{c.W}D{c.D}g{c.Hq // c.Hkv}t{c.dtype}")
def test_small_random_step_sequences(cfg, mode):
    say(f"small sweep {cfg} mode={mode}")
    rng = np.random.default_rng(cfg.seed)
    run = Lockstep(cfg, mode=mode)
    T = 0
    for _ in range(14):
        S = int(rng.choice([1, 1, 1, 2, 3, int(rng.integers(1, 2 * cfg.C + 2))]))
        run.step([T] * cfg.B, S)
        T += S
    say(f"  worst scaled error {run.worst:.3g}")


@pytest.mark.parametrize("mode", ["shared", "separate"])
def test_ragged_batch_with_bias(mode):
    """Items at different lengths in one multi-token step, with an absolute-
    column bias whose invisible columns are NaN (so reading one shows)."""
    cfg = Cfg(B=4, Hq=8, Hkv=2, D=64, C=45, W=40, seed=19, dtype=synth.F16)
    syn = cfg.synth()
    vers = Versions(4)
    P0 = np.array([0, 37, 90, 140])
    K, V = seeded_cache(cfg, syn, P0, vers)
    run = Lockstep(cfg, mode=mode, K=K, V=V, vers=vers)
    P = P0.copy()
    for S in [8, 1, 5, 8, 3, 1, 8]:
        total = int((P + S).max())
        bias = syn.bias_f32(np.arange(4), P, S, total)
        j = np.arange(total)[None, None, None, :]
        p = (P[:, None, None, None] + np.arange(S)[None, None, :, None])
        vis = (j <= p) & (j > p - cfg.W)
        bias = synth.to_storage(np.where(vis, bias, np.float32(np.nan)), cfg.dtype)
        run.step(P, S, bias=bias, total=total)
        P = P + S
    say(f"  worst scaled error {run.worst:.3g}")


def test_bias_broadcast_dims():
    cfg = Cfg(B=2, Hq=4, Hkv=2, D=8, C=12, W=6, seed=20)
    syn = cfg.synth()
    vers = Versions(2)
    P = np.array([9, 17])
    K, V = seeded_cache(cfg, syn, P, vers)
    for bb, bh in [(0, 0), (1, 0), (0, 1)]:
        run = Lockstep(cfg, K=K, V=V, vers=vers)
        shape = (2 if bb else 1, 4 if bh else 1, 3, 20)
        bias = np.random.default_rng(bb * 2 + bh).normal(0, 0.5, shape).astype(np.float32)
        run.step(P, 3, bias=bias, total=20, bias_bcast=(bb, bh))


# ---------------------------------------------------------------------------
# The pages' decode shape (64 Q / 8 KV heads x 64, fp32, W=128, C=384) with a
# 512-token prefill and decode steps across the first compaction (T=642).
def test_pages_shape_prompt512():
    cfg = Cfg(B=1, Hq=64, Hkv=8, D=64, C=384, W=128, seed=1002, scale=0.125)
    say("pages' shape, prompt 512")
    run = Lockstep(cfg)
    run.step([0], 512)
    for T in range(513, 513 + 140):
        run.step([T - 1], 1, check_regen=(T % 16 == 0 or T in (641, 642, 643)))
    say(f"  worst scaled error {run.worst:.3g}")


# Small-slack compaction stress: C = W + 8 (G = 9), prefill 512 then 400
# decodes: 45 compaction events, each an overlapping in-place move.
def test_small_slack_400_decodes():
    cfg = Cfg(B=1, Hq=64, Hkv=8, D=64, C=136, W=128, seed=1003)
    say("small slack, 512 + 400")
    run = Lockstep(cfg)
    run.step([0], 512)
    events = 0
    for T in range(513, 913):
        _, _, plan = run.step([T - 1], 1, check_regen=(T % 9 == 0))
        events += int(plan[0, 5] > 0)
    assert events == 45
    say(f"  worst scaled error {run.worst:.3g}")


# The capacity sweep's tightest points at the pages' decode shape: C = W
# (gap 1, a compaction on every decode step) and C = W + 4 (gap 5), after a
# 2048-token prompt, 300 decodes, every step compared ("[CPU] Add windowed kv
# cache for GQA", Performance Results: decode latency against capacity).
@pytest.mark.parametrize("slack", [0, 4])
def test_pages_shape_tight_capacity(slack):
    cfg = Cfg(B=1, Hq=64, Hkv=8, D=64, C=128 + slack, W=128, seed=1010 + slack, scale=0.125)
    say(f"pages' shape, C = W + {slack}, prompt 2048 + 300 decodes")
    run = Lockstep(cfg, vers=Versions(1, n=2400))
    run.step([0], 2048)
    events = 0
    for T in range(2049, 2349):
        _, _, plan = run.step([T - 1], 1, check_regen=(T % 7 == 0))
        events += int(plan[0, 5] > 0)
    assert events == (300 if slack == 0 else 60)
    say(f"  worst scaled error {run.worst:.3g}, {events} compactions")


# Compactions with a long gap on the 8-wave staged decode kernel, one
# workgroup per (item, KV head): the surviving rows are stored at their new
# place while attention reads them, behind a barrier every 2^k rounds of the
# waves' stages (the gap holds at least one round).  Each item starts a few
# steps before its next compaction (past lengths seeded in the contract
# layout), so every item compacts once or twice; every output, every resident
# row byte for byte, the poison of unwritten rows and the canaries are checked
# after every step.  Shapes: the gap exactly one round (a barrier after every
# round), two and more rounds, a window that is not a whole number of rounds,
# fp32 / fp16 / bf16 at the stage shapes the variant is built for, and
# two-token steps on a one-tile slice.
FUSED_MOVE = [
    (Cfg(B=8, Hq=32, Hkv=8, D=128, C=327, W=200, seed=151, dtype=synth.BF16), [1]),
    (Cfg(B=8, Hq=32, Hkv=8, D=128, C=600, W=200, seed=152, dtype=synth.BF16, softcap=30.0),
     [1]),
    (Cfg(B=16, Hq=32, Hkv=8, D=128, C=1300, W=1000, seed=153, dtype=synth.BF16), [1]),
    (Cfg(B=8, Hq=32, Hkv=8, D=64, C=400, W=230, seed=154, dtype=synth.F32), [1]),
    (Cfg(B=2, Hq=2, Hkv=2, D=64, C=495, W=240, seed=155, dtype=synth.F16), [1, 2]),
    (Cfg(B=32, Hq=16, Hkv=2, D=32, C=313, W=250, seed=156, dtype=synth.F32), [1]),
    # 8-bit caches at the same shapes: the kernel that moves rows after
    # attention (long gaps, one 8-wave workgroup per slice)
    (Cfg(B=8, Hq=32, Hkv=8, D=128, C=327, W=200, seed=157, dtype=synth.BF16, kv_int8=True,
         k_scale=0.03, v_scale=0.02), [1]),
    (Cfg(B=8, Hq=32, Hkv=8, D=64, C=400, W=230, seed=158, dtype=synth.F16, kv_fp8=True,
         k_scale=0.05, v_scale=0.04, softcap=30.0), [1]),
]


@pytest.mark.parametrize("cfg,steps", FUSED_MOVE,
                         ids=lambda c: f"W{c.W}G{c.C - c.W + 1}D{c.D}t{c.dtype}"
                         f"{'i8' if c.kv_int8 else 'f8' if c.kv_fp8 else ''}"
                         if isinstance(c, Cfg) else "")
def test_long_gap_compaction_moves_while_reading(cfg, steps):
    G = cfg.C - cfg.W + 1
    syn = cfg.synth()
    # item b compacts on its step offs[b] + 1 (its past length reaches C + G);
    # the small batches run on through a second compaction
    offs = [(3 + 11 * b) % min(G, 40) for b in range(cfg.B)]
    P = np.array([cfg.C + G - 1 - o for o in offs], dtype=np.int64)
    n = max(offs) + 2 + (G if cfg.B * cfg.Hq <= 256 else 0)
    vers = Versions(cfg.B, n=int(P.max()) + 2 * n + 8)
    K, V = seeded_cache(cfg, syn, P, vers)
    run = Lockstep(cfg, K=K, V=V, vers=vers)
    say(f"long-gap compaction {cfg}: G={G}, {n} steps from P={list(P[:4])}")
    events = 0
    for i in range(n):
        S = steps[i % len(steps)]
        _, _, plan = run.step(P, S, check_regen=(i % 5 == 0))
        events += int((plan[:, 5] > 0).sum())
        P = P + S
    say(f"  {events} compaction events, worst scaled error {run.worst:.3g}")
    assert events >= cfg.B


# Rows wider than 256 bytes: fp32 at head size 128 and 256, bf16 at 256.
# Steps of few query rows go to the generic split kernel (whole slices, and
# key splits merged by the step tail over a long window); fp32 D = 128 and
# bf16 D = 256 multi-token steps take the matrix-core kernel's 512-byte rows;
# fp32 D = 256 multi-token steps stay on the split kernel.
WIDE = [
    Cfg(B=2, Hq=4, Hkv=2, D=128, C=40, W=33, seed=141, dtype=synth.F32),
    Cfg(B=2, Hq=8, Hkv=2, D=256, C=30, W=24, seed=142, dtype=synth.F32, softcap=20.0),
    Cfg(B=2, Hq=4, Hkv=1, D=256, C=36, W=30, seed=143, dtype=synth.BF16, sink_std=1.0),
    Cfg(B=3, Hq=12, Hkv=3, D=128, C=70, W=64, seed=144, dtype=synth.F32, rotary=1),
    Cfg(B=1, Hq=8, Hkv=8, D=256, C=20, W=17, seed=145, dtype=synth.BF16, softcap=30.0,
        rotary=0),
]


@pytest.mark.parametrize("mode", ["shared", "separate"])
@pytest.mark.parametrize("cfg", WIDE, ids=lambda c: f"D{c.D}t{c.dtype}g{c.Hq // c.Hkv}")
def test_wide_rows_random_steps(cfg, mode):
    say(f"wide rows {cfg} mode={mode}")
    rng = np.random.default_rng(cfg.seed)
    run = Lockstep(cfg, mode=mode)
    T = 0
    for S in [1, 3, 1, 16, 1, 2, 33, 1, 17, int(rng.integers(1, 2 * cfg.C + 2)), 1, 5,
              2 * cfg.C + 1, 1]:
        run.step([T] * cfg.B, S)
        T += S
    say(f"  worst scaled error {run.worst:.3g}")


@pytest.mark.parametrize("mode", ["shared", "separate"])
@pytest.mark.parametrize("dtype,D", [(synth.F32, 128), (synth.F32, 256), (synth.BF16, 256)],
                         ids=["f32_128", "f32_256", "bf16_256"])
def test_wide_rows_key_splits_with_bias(dtype, D, mode):
    """A long window over one slice: key splits on the split kernel (short
    steps) or the matrix-core kernel (fp32 D=128 and bf16 D=256 chunks),
    merged by the step tail; a NaN bias outside the visible band."""
    cfg = Cfg(B=1, Hq=4, Hkv=1, D=D, C=1600, W=1500, seed=146 + D, dtype=dtype, softcap=40.0)
    syn = cfg.synth()
    vers = Versions(1)
    P0 = np.array([1700])
    K, V = seeded_cache(cfg, syn, P0, vers)
    run = Lockstep(cfg, mode=mode, K=K, V=V, vers=vers)
    P = P0.copy()
    for S, with_bias in [(1, False), (3, True), (40, True), (1, True), (16, False)]:
        total = int((P + S).max())
        bias = _bias_nan_outside(cfg, syn, P, S, total) if with_bias else None
        run.step(P, S, bias=bias, total=total)
        P = P + S
    say(f"  worst scaled error {run.worst:.3g}")


@pytest.mark.parametrize("mode", ["shared", "separate"])
@pytest.mark.parametrize("code", ["int8", "fp8"])
def test_eight_bit_cache_fp32_head_size_256(code, mode):
    """fp32 queries at head size 256 over an 8-bit cache: every step of up
    to 16 tokens on the 8-bit staged kernel (16 included); longer steps are
    refused before any launch."""
    import sliding_window_gqa_02_amd as sw
    cfg = Cfg(B=2, Hq=4, Hkv=2, D=256, C=40, W=33, seed=148, kv_int8=code == "int8",
              kv_fp8=code == "fp8", k_scale=0.03, v_scale=0.02)
    run = Lockstep(cfg, mode=mode)
    T = 0
    for S in [16, 1, 3, 1, 15, 1, 16, 2, 1, 8, 16, 1]:
        run.step([T] * cfg.B, S)
        T += S
    say(f"  worst scaled error {run.worst:.3g}")
    t = torch.zeros(1 << 16, dtype=torch.float32, device="cuda:0")
    ws = torch.zeros(1 << 16, dtype=torch.int32, device="cuda:0")
    seq = torch.full((2,), T + 16, dtype=torch.int32, device="cuda:0")
    p = sw.make_params(2, 17, 4, 2, 256, 40, 33, T + 17, synth.F32, **cfg.cache_params())
    assert sw.forward_status(p, t, t, t, t, t, seq, None, t, t, t, ws) == sw.ERR_UNSUPPORTED
    torch.cuda.synchronize()


# One workspace, sized for a long-window key-split step (partials), then
# reused for decode steps of a few-slice shape whose query tiles share each
# slice and compact through the per-slice counters: the counters sit in the
# fixed workspace header, never under another call's partials.
def test_workspace_reuse_split_then_counted_compaction():
    big = Cfg(B=1, Hq=4, Hkv=1, D=128, C=1600, W=1500, seed=37, dtype=synth.BF16)
    say("workspace reuse: key splits, then counted compaction")
    import sliding_window_gqa_02_amd as sw
    p_big = sw.make_params(1, 1, 4, 1, 128, 1600, 1500, 3001, synth.BF16)
    small = Cfg(B=1, Hq=16, Hkv=2, D=64, C=20, W=12, seed=38)
    ws_bytes = max(sw.workspace_size(p_big), 1 << 16)
    run_big = Lockstep(big)
    run_big.gpu.ws = torch.zeros(ws_bytes // 4, dtype=torch.int32, device="cuda:0")
    run_big.gpu.ws_bytes = ws_bytes
    sw.workspace_init(run_big.gpu.ws)
    run_big.step([0], 1500)
    run_big.step([1500], 1)   # decode over a 1500-key window: key splits + combine
    run = Lockstep(small)
    run.gpu.ws, run.gpu.ws_bytes = run_big.gpu.ws, ws_bytes
    run.step([0], 15)
    events = 0
    for T in range(16, 60):
        _, _, plan = run.step([T - 1], 1)
        events += int(plan[0, 5] > 0)
    assert events >= 4
    say(f"  worst scaled error {run.worst:.3g}, {events} compactions")


# ---------------------------------------------------------------------------
def test_invalid_items_flagged_zeroed_untouched():
    import sliding_window_gqa_02_amd as sw
    cfg = Cfg(B=3, Hq=4, Hkv=2, D=8, C=6, W=4, seed=21)
    syn = cfg.synth()
    vers = Versions(3)
    P = np.array([5, 5, 5])
    K, V = seeded_cache(cfg, syn, P, vers)
    from tests.gpu_backend import GpuBackend
    g = GpuBackend(cfg, K, V)
    q, k, v = step_inputs(cfg, syn, P, 2, vers)
    before = g.present_host()
    st, out = g.step(2, np.array([6, 0, 6], np.int32), q, k, v, total=7, poison=False)
    assert st == sw.ERR_DEVICE_INPUT
    assert np.all(out[1] == 0)
    after = g.present_host()
    assert np.array_equal(after[0][1].view(np.uint8), before[0][1].view(np.uint8))
    # the other items were computed
    o = __import__("tests.scenario", fromlist=["OracleBackend"]).OracleBackend(cfg, K, V)
    st_o, out_o, _ = o.step(2, np.array([6, 0, 6], np.int32), q, k, v, total=7)
    assert st_o == 4
    assert np.allclose(out[0], out_o[0], rtol=1e-5, atol=1e-5)
    # status cleared by the read
    st, _ = g.step(2, np.array([6, 6, 6], np.int32), q, k, v, total=7, poison=False)
    assert st == sw.OK


def test_host_errors_return_before_launch():
    import sliding_window_gqa_02_amd as sw
    t = torch.zeros(4096, dtype=torch.float32, device="cuda:0")
    ws = torch.zeros(1024, dtype=torch.int32, device="cuda:0")
    seq = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    bad = [
        sw.make_params(1, 1, 3, 2, 8, 6, 4, 8),     # Hq % Hkv
        sw.make_params(1, 1, 2, 2, 8, 6, 7, 8),     # W > C
        sw.make_params(1, 1, 2, 2, 8, 6, 0, 8),     # W < 1
        sw.make_params(1, 0, 2, 2, 8, 6, 4, 8),     # S < 1
    ]
    for p in bad:
        assert sw.forward_status(p, t, t, t, t, t, seq, None, t, t, t, ws) == sw.ERR_ARG
    p = sw.make_params(1, 1, 2, 2, 12, 6, 4, 8)     # unsupported head size
    assert sw.forward_status(p, t, t, t, t, t, seq, None, t, t, t, ws) == sw.ERR_UNSUPPORTED
    p = sw.make_params(1, 1, 2, 2, 8, 6, 4, 8)
    assert sw.forward_status(p, t, t, t, t[16:], t[16:], seq, None, t, t[32:], t[32:], ws) == sw.ERR_ALIAS
    assert sw.forward_status(p, t, t, t, t, t, seq, None, t, t, t, ws, workspace_bytes=16) == sw.ERR_ARG
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# Multi-token steps (S >= 16) run on the matrix-core kernel.
def _bias_nan_outside(cfg, syn, P, S, total):
    bias = syn.bias_f32(np.arange(len(P)), P, S, total)
    j = np.arange(total)[None, None, None, :]
    p = np.asarray(P)[:, None, None, None] + np.arange(S)[None, None, :, None]
    vis = (j <= p) & (j > p - cfg.W)
    return synth.to_storage(np.where(vis, bias, np.float32(np.nan)), cfg.dtype)


CHUNK = [
    Cfg(B=3, Hq=8, Hkv=2, D=64, C=110, W=100, seed=31, dtype=synth.F32, softcap=20.0),
    Cfg(B=3, Hq=8, Hkv=2, D=128, C=110, W=100, seed=32, dtype=synth.F16),
    Cfg(B=2, Hq=12, Hkv=3, D=128, C=90, W=64, seed=33, dtype=synth.BF16, softcap=30.0),
    Cfg(B=2, Hq=4, Hkv=4, D=32, C=70, W=70, seed=34, dtype=synth.F16),
    Cfg(B=1, Hq=16, Hkv=2, D=16, C=48, W=40, seed=35, dtype=synth.F32),
]


@pytest.mark.parametrize("mode", ["shared", "separate"])
@pytest.mark.parametrize("cfg", CHUNK, ids=lambda c: f"D{c.D}g{c.Hq // c.Hkv}t{c.dtype}cap{int(c.softcap)}")
def test_chunked_steps_ragged_bias(cfg, mode):
    say(f"chunked {cfg} mode={mode}")
    syn = cfg.synth()
    vers = Versions(cfg.B)
    P0 = np.array([0, 57, 133][:cfg.B])
    K, V = seeded_cache(cfg, syn, P0, vers)
    run = Lockstep(cfg, mode=mode, K=K, V=V, vers=vers)
    P = P0.copy()
    for S, with_bias in [(32, True), (17, False), (48, True), (150, False), (16, True), (1, False)]:
        total = int((P + S).max())
        bias = _bias_nan_outside(cfg, syn, P, S, total) if with_bias else None
        run.step(P, S, bias=bias, total=total)
        P = P + S
    say(f"  worst scaled error {run.worst:.3g}")


# Wave groups of the chunk kernel (tiles of at most 32 query rows, 16-bit):
# 256 slices, so one key split per slice and up to 10 blocks per split --
# several staging rounds, the last with groups that have no block.  With 4
# query heads per KV head, S = 8 takes the groups, S = 16 the 64-row tiles
# and S = 4 the staged decode kernel; with one, S = 16 / 24 / 32 give tiles
# of 16 / 24 / 32 rows (group waves without rows, or with some).
GROUPS = [
    (Cfg(B=16, Hq=64, Hkv=16, D=64, C=320, W=300, seed=36, dtype=synth.F16),
     [(8, True), (8, False), (4, True), (16, False), (8, True), (4, False), (8, False), (8, True)]),
    (Cfg(B=16, Hq=64, Hkv=16, D=128, C=310, W=290, seed=37, dtype=synth.BF16, softcap=25.0),
     [(8, True), (16, False), (8, False), (8, True), (4, False), (8, True)]),
    (Cfg(B=16, Hq=16, Hkv=16, D=64, C=300, W=280, seed=38, dtype=synth.F16),
     [(16, True), (24, False), (32, True), (16, False), (24, True)]),
]


@pytest.mark.parametrize("mode", ["shared", "separate"])
@pytest.mark.parametrize("cfg,steps", GROUPS,
                         ids=lambda c: f"D{c.D}g{c.Hq // c.Hkv}t{c.dtype}" if isinstance(c, Cfg) else "")
def test_chunk_wave_groups_many_rounds(cfg, steps, mode):
    say(f"wave groups {cfg} mode={mode}")
    syn = cfg.synth()
    vers = Versions(cfg.B)
    P0 = np.array([cfg.W - 40 + 7 * b for b in range(cfg.B)], dtype=np.int64)
    K, V = seeded_cache(cfg, syn, P0, vers)
    run = Lockstep(cfg, mode=mode, K=K, V=V, vers=vers)
    P = P0.copy()
    events = 0
    for S, with_bias in steps:
        total = int((P + S).max())
        bias = _bias_nan_outside(cfg, syn, P, S, total) if with_bias else None
        _, _, plan = run.step(P, S, bias=bias, total=total)
        events += int((plan[:, 5] > 0).sum())
        P = P + S
    say(f"  {events} compaction events, worst scaled error {run.worst:.3g}")
    assert events > 0


def test_bias_rows_shorter_than_a_load_group():
    """Bias rows of 2, 9 and 13 entries: the chunk kernel reads bias in groups
    of 8 entries clamped to the row's end (shifted back when computed: by 7
    and 3 entries here), and a step with rows of fewer than 8 entries goes to
    the staged decode kernel."""
    cfg = Cfg(B=2, Hq=32, Hkv=2, D=64, C=12, W=10, seed=37, dtype=synth.F16)
    syn = cfg.synth()
    vers = Versions(cfg.B)
    run = Lockstep(cfg, vers=vers)
    P = np.array([0, 0])
    for S in [2, 7, 4]:
        total = int((P + S).max())
        run.step(P, S, bias=_bias_nan_outside(cfg, syn, P, S, total), total=total)
        P = P + S
    say(f"  worst scaled error {run.worst:.3g}")


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16], ids=["f32", "bf16"])
def test_positions_near_int32_limit(dtype):
    """Lengths up to 2^31 - 1 (seqlens_k near the int32 limit, the planner's
    division at the top of its range): decode, short multi-token and chunked
    steps, with compactions, from caches holding the contract layout."""
    cfg = Cfg(B=2, Hq=8, Hkv=2, D=64, C=40, W=33, seed=38, dtype=dtype, softcap=20.0)
    syn = cfg.synth()
    top = 2**31 - 1
    vers = Versions(cfg.B, n=4096, base=top - 4000)
    P0 = np.array([top - 60, top - 41])
    K, V = seeded_cache(cfg, syn, P0, vers)
    run = Lockstep(cfg, K=K, V=V, vers=vers)
    P = P0.copy()
    for S in [1, 2, 1, 17, 1, 3, 1, 9, 1, 1]:
        run.step(P, S, total=int((P + S).max()))
        P = P + S
    assert int(P.max()) <= top
    say(f"  worst scaled error {run.worst:.3g}")


def test_chunk_key_splits_long_window():
    """Few (item, KV head) slices and a long window: the chunk kernel splits
    the key band across workgroups and a merge kernel combines them."""
    cfg = Cfg(B=1, Hq=4, Hkv=1, D=128, C=1600, W=1500, seed=36, dtype=synth.BF16, softcap=50.0)
    syn = cfg.synth()
    vers = Versions(1)
    P0 = np.array([1700])
    K, V = seeded_cache(cfg, syn, P0, vers)
    run = Lockstep(cfg, K=K, V=V, vers=vers)
    P = P0.copy()
    for S in [64, 64, 1, 40]:
        run.step(P, S)
        P = P + S
    say(f"  worst scaled error {run.worst:.3g}")


# Key splits of a one-tile chunk step that move the surviving rows as they
# read them (16-bit cache, shared buffer): each split stores its kept rows at
# their new place, the first `shift` of them (whose new place lies in the
# previous split's part) through a stash that the step tail stores.  Shapes:
# verify and chunked-prefill steps at gap 9 with bias, gap 1 (every step
# compacts by S), 512-byte rows, shifts over the 64-row stash (66 rows: the
# step tail moves every row), and compactions that keep rows below the key
# band (the step tail moves every row); ragged items compact on different
# steps.
SPLIT_MOVE = [
    (Cfg(B=2, Hq=8, Hkv=2, D=128, C=508, W=500, seed=161, dtype=synth.F16), [32, 8, 8, 32, 8], True),
    (Cfg(B=2, Hq=16, Hkv=2, D=64, C=300, W=300, seed=162, dtype=synth.BF16, softcap=30.0),
     [16, 8, 16], False),
    (Cfg(B=1, Hq=8, Hkv=2, D=256, C=419, W=400, seed=163, dtype=synth.F16), [16, 8], False),
    (Cfg(B=2, Hq=4, Hkv=2, D=128, C=432, W=400, seed=164, dtype=synth.BF16), [64, 16, 64], False),
    (Cfg(B=2, Hq=8, Hkv=2, D=64, C=329, W=300, seed=165, dtype=synth.F16), [16, 20], True),
    # shift = 64, the rows set aside per split (the splits move), and 65,
    # one more (the step tail moves)
    (Cfg(B=2, Hq=8, Hkv=2, D=128, C=463, W=400, seed=166, dtype=synth.F16), [32, 8, 64], True),
    (Cfg(B=2, Hq=8, Hkv=2, D=128, C=464, W=400, seed=167, dtype=synth.BF16), [16, 48], False),
]


@pytest.mark.parametrize("cfg,steps,with_bias", SPLIT_MOVE,
                         ids=lambda c: f"W{c.W}G{c.C - c.W + 1}D{c.D}t{c.dtype}"
                         if isinstance(c, Cfg) else "")
def test_chunk_key_splits_move_while_reading(cfg, steps, with_bias):
    import sliding_window_gqa_02_amd as sw
    G = cfg.C - cfg.W + 1
    if cfg.D <= 128:
        # the stash is planned for gaps up to 64 rows: the 16-bit step's
        # workspace then exceeds that of the fp32 step (same kernel and
        # partials, no stash) by it; beyond, the two are equal
        ws = [sw.workspace_size(sw.make_params(cfg.B, steps[0], cfg.Hq, cfg.Hkv, cfg.D, cfg.C,
                                               cfg.W, cfg.C + 4 * G, dt, 0.0, 0.0, 1, 1))
              for dt in (cfg.dtype, synth.F32)]
        assert (ws[0] > ws[1] > 0) if G <= 64 else (ws[0] == ws[1] > 0), ws
    syn = cfg.synth()
    vers = Versions(cfg.B, n=cfg.C + 40 * max(steps) + 64)
    P = np.array([cfg.C - 5 - 7 * b for b in range(cfg.B)], dtype=np.int64)
    K, V = seeded_cache(cfg, syn, P, vers)
    run = Lockstep(cfg, K=K, V=V, vers=vers)
    n = 4 * len(steps) + 4
    say(f"split-move {cfg}: G={G}, {n} steps from P={list(P)}")
    events = 0
    for i in range(n):
        S = steps[i % len(steps)]
        total = int((P + S).max())
        bias = _bias_nan_outside(cfg, syn, P, S, total) if with_bias and i % 2 == 0 else None
        _, _, plan = run.step(P, S, bias=bias, total=total, check_regen=(i % 3 == 0))
        events += int((plan[:, 5] > 0).sum())
        P = P + S
    say(f"  {events} compaction events, worst scaled error {run.worst:.3g}")
    assert events >= 2 * cfg.B


# ---------------------------------------------------------------------------
# Softmax sink (head_sink per query head, or smooth_softmax's logit 0) on
# every output path: whole-slice decode and MFMA chunks (fp32, bf16), the
# generic split kernel (D = 256), and key splits merged by the step tail.
SINK = [
    Cfg(B=2, Hq=8, Hkv=2, D=64, C=40, W=33, seed=41, sink_std=1.0),
    Cfg(B=2, Hq=16, Hkv=2, D=128, C=70, W=64, seed=42, dtype=synth.BF16, softcap=30.0,
        smooth=True),
    Cfg(B=1, Hq=4, Hkv=4, D=256, C=20, W=17, seed=43, dtype=synth.F16, sink_std=2.0),
]


@pytest.mark.parametrize("cfg", SINK, ids=lambda c: f"D{c.D}t{c.dtype}smooth{int(c.smooth)}")
def test_softmax_sink_random_steps(cfg):
    say(f"softmax sink {cfg}")
    rng = np.random.default_rng(cfg.seed)
    run = Lockstep(cfg)
    T = 0
    for _ in range(12):
        S = int(rng.choice([1, 1, 1, 2, 8, int(rng.integers(1, 2 * cfg.C + 2))]))
        run.step([T] * cfg.B, S)
        T += S
    say(f"  worst scaled error {run.worst:.3g}")


def test_softmax_sink_key_splits():
    cfg = Cfg(B=1, Hq=4, Hkv=1, D=128, C=1600, W=1500, seed=44, dtype=synth.BF16,
              sink_std=1.0)
    say("softmax sink with key splits")
    syn = cfg.synth()
    vers = Versions(1)
    P0 = np.array([1700])
    K, V = seeded_cache(cfg, syn, P0, vers)
    run = Lockstep(cfg, K=K, V=V, vers=vers)
    P = P0.copy()
    for S in [64, 1, 1, 40]:
        run.step(P, S)
        P = P + S
    say(f"  worst scaled error {run.worst:.3g}")


# ---------------------------------------------------------------------------
# Rotary embedding of the query and new key rows (cos / sin tables, default
# positions P + i or explicit position_ids) on every kernel path: fused into
# the staged decode kernel (D = 32, 64, 128; in-kernel append and compaction,
# or the step tail in separate-buffer mode and after key splits), and as a
# pass of its own before the generic split kernel (D = 256) and the MFMA
# chunks.  The cache stores rotated keys, compared byte for byte with the
# oracle's.
ROTARY = [
    Cfg(B=2, Hq=8, Hkv=2, D=64, C=40, W=33, seed=51, rotary=0),
    Cfg(B=2, Hq=16, Hkv=2, D=128, C=70, W=64, seed=52, dtype=synth.BF16, rotary=1,
        softcap=30.0),
    Cfg(B=1, Hq=4, Hkv=4, D=256, C=20, W=17, seed=53, dtype=synth.F16, rotary=0),
    Cfg(B=3, Hq=8, Hkv=2, D=128, C=110, W=100, seed=54, dtype=synth.F16, rotary=1,
        sink_std=1.0),
    Cfg(B=2, Hq=4, Hkv=1, D=32, C=48, W=40, seed=55, dtype=synth.F32, rotary=1),
    Cfg(B=2, Hq=8, Hkv=2, D=64, C=40, W=33, seed=58, dtype=synth.BF16, rotary=0),
    Cfg(B=2, Hq=4, Hkv=2, D=32, C=30, W=20, seed=59, dtype=synth.F16, rotary=1),
]


@pytest.mark.parametrize("mode", ["shared", "separate"])
@pytest.mark.parametrize("explicit", [False, True], ids=["default_pos", "position_ids"])
@pytest.mark.parametrize("cfg", ROTARY, ids=lambda c: f"D{c.D}t{c.dtype}il{c.rotary}")
def test_rotary_random_steps(cfg, explicit, mode):
    say(f"rotary {cfg} position_ids={explicit} mode={mode}")
    rng = np.random.default_rng(cfg.seed)
    run = Lockstep(cfg, mode=mode)
    T = np.zeros(cfg.B, np.int64)
    off = rng.integers(0, 9, size=cfg.B)       # per-item offset (left padding)
    for _ in range(12):
        S = int(rng.choice([1, 1, 2, 8, 16, 33, int(rng.integers(1, 2 * cfg.C + 2))]))
        pos = (T[:, None] + np.arange(S)[None, :] + off[:, None]) if explicit else None
        run.step(T, S, position_ids=pos)
        T = T + S
    say(f"  worst scaled error {run.worst:.3g}")


def test_rotary_chunk_key_splits():
    cfg = Cfg(B=1, Hq=4, Hkv=1, D=128, C=1600, W=1500, seed=56, dtype=synth.BF16, rotary=0)
    say("rotary with key splits")
    syn = cfg.synth()
    vers = Versions(1)
    P0 = np.array([1700])
    K, V = seeded_cache(cfg, syn, P0, vers)
    run = Lockstep(cfg, K=K, V=V, vers=vers)
    P = P0.copy()
    for S in [64, 1, 40]:
        run.step(P, S)
        P = P + S
    say(f"  worst scaled error {run.worst:.3g}")


@pytest.mark.parametrize("mode", ["shared", "separate"])
@pytest.mark.parametrize("D", [16, 64], ids=["prepass", "fused"])
def test_rotary_position_outside_tables_flags_item(D, mode):
    """An item whose position reaches past the tables is skipped like an
    out-of-range length: flagged, zero output, its cache rows untouched; the
    other items are computed."""
    import sliding_window_gqa_02_amd as sw
    from tests.gpu_backend import GpuBackend
    from tests.scenario import OracleBackend
    cfg = Cfg(B=3, Hq=4, Hkv=2, D=D, C=12, W=8, seed=57, rotary=0, rot_rows=16)
    syn = cfg.synth()
    vers = Versions(3)
    P = np.array([5, 5, 5])
    K, V = seeded_cache(cfg, syn, P, vers)
    g = GpuBackend(cfg, K, V, mode=mode)
    q, k, v = step_inputs(cfg, syn, P, 3, vers)
    seq = np.array([7, 7, 7], np.int32)
    pos = np.array([[5, 6, 7], [14, 15, 16], [-1, 0, 1]])   # items 1 and 2 invalid
    before = g.present_host()
    st, out = g.step(3, seq, q, k, v, total=8, poison=False, position_ids=pos)
    assert st == sw.ERR_DEVICE_INPUT
    assert np.all(out[1] == 0) and np.all(out[2] == 0)
    after = g.present_host()
    for b in (1, 2):
        if mode == "shared":
            assert np.array_equal(after[0][b].view(np.uint8), before[0][b].view(np.uint8))
            assert np.array_equal(after[1][b].view(np.uint8), before[1][b].view(np.uint8))
        else:  # the separate present buffer keeps the NaN it was filled with
            from tests.scenario import as_f64
            assert np.isnan(as_f64(after[0][b], cfg.dtype)).all()
            assert np.isnan(as_f64(after[1][b], cfg.dtype)).all()
    o = OracleBackend(cfg, K, V)
    st_o, out_o, _ = o.step(3, seq, q, k, v, total=8, position_ids=pos)
    assert st_o == 4
    assert np.allclose(out[0], out_o[0], rtol=1e-5, atol=1e-5)
    L = oracle.resident_length(8, cfg.C, cfg.W)
    assert np.array_equal(after[0][0, :, :L].view(np.uint8), o.K[0, :, :L].view(np.uint8))
    # the same step with positions inside the tables succeeds
    st, _ = g.step(3, seq, q, k, v, total=8, poison=False,
                   position_ids=np.array([[5, 6, 7], [5, 6, 7], [5, 6, 7]]))
    assert st == sw.OK


# ---------------------------------------------------------------------------
# int8 cache (kv_cache_type 1): per-tensor scales, new rows quantized on the
# way in, every row read dequantized.  Steps of fewer than 16 tokens on the
# int8 staged kernel (whole slice, query tiles with the counted compaction,
# key splits merged by the step tail), both buffer modes; cache codes
# compared byte for byte with the oracle's.
Q8 = [
    Cfg(B=2, Hq=8, Hkv=2, D=64, C=40, W=33, seed=61, kv_int8=True),
    Cfg(B=2, Hq=16, Hkv=2, D=128, C=70, W=64, seed=62, dtype=synth.BF16, softcap=30.0,
        kv_int8=True, k_scale=0.03, v_scale=0.02),
    Cfg(B=1, Hq=4, Hkv=4, D=256, C=20, W=17, seed=63, dtype=synth.F16, kv_int8=True),
    Cfg(B=3, Hq=4, Hkv=2, D=32, C=30, W=20, seed=64, dtype=synth.F16, kv_int8=True,
        sink_std=1.0),
    Cfg(B=1, Hq=2, Hkv=1, D=16, C=12, W=9, seed=65, kv_int8=True, smooth=True),
    Cfg(B=2, Hq=8, Hkv=2, D=64, C=40, W=33, seed=66, dtype=synth.BF16, kv_int8=True,
        rotary=0),
    Cfg(B=3, Hq=8, Hkv=2, D=128, C=90, W=70, seed=67, dtype=synth.F16, softcap=40.0,
        kv_int8=True, k_scale=0.03, v_scale=0.05),
]


@pytest.mark.parametrize("mode", ["shared", "separate"])
@pytest.mark.parametrize("cfg", Q8, ids=lambda c: f"D{c.D}t{c.dtype}g{c.Hq // c.Hkv}rot{c.rotary}")
def test_int8_cache_random_steps(cfg, mode):
    say(f"int8 cache {cfg} mode={mode}")
    rng = np.random.default_rng(cfg.seed)
    run = Lockstep(cfg, mode=mode)
    T = 0
    for _ in range(16):
        S = int(rng.choice([1, 1, 1, 2, 3, 5, 8, 15, 16, 33, int(rng.integers(1, 2 * cfg.C + 2))]))
        run.step([T] * cfg.B, S)
        T += S
    say(f"  worst scaled error {run.worst:.3g}")


def test_int8_cache_ragged_bias_and_key_splits():
    """Items at different lengths with an absolute-column bias, then a long
    window over few slices (key splits, merged and written back by the step
    tail, which quantizes the new rows)."""
    cfg = Cfg(B=3, Hq=8, Hkv=2, D=64, C=45, W=40, seed=67, dtype=synth.F16, kv_int8=True)
    syn = cfg.synth()
    vers = Versions(3)
    P0 = np.array([0, 37, 90])
    K, V = seeded_cache(cfg, syn, P0, vers)
    run = Lockstep(cfg, K=K, V=V, vers=vers)
    P = P0.copy()
    for S in [8, 1, 5, 1, 3]:
        total = int((P + S).max())
        run.step(P, S, bias=_bias_nan_outside(cfg, syn, P, S, total), total=total)
        P = P + S
    long = Cfg(B=1, Hq=4, Hkv=1, D=128, C=1600, W=1500, seed=68, dtype=synth.BF16,
               kv_int8=True)
    syn = long.synth()
    vers = Versions(1)
    P0 = np.array([1700])
    K, V = seeded_cache(long, syn, P0, vers)
    for mode in ("shared", "separate"):
        run = Lockstep(long, mode=mode, K=K, V=V, vers=vers)
        P = P0.copy()
        for S in [1, 4, 1, 15]:
            run.step(P, S)
            P = P + S
    say(f"  worst scaled error {run.worst:.3g}")


@pytest.mark.parametrize("mode", ["shared", "separate"])
def test_int8_cache_multi_token_steps(mode):
    """Steps of 16 or more tokens over an int8 cache take the matrix-core
    kernel on codes: a staged prefill (S > C), chunks with a bias, verify
    steps, then a long window over few slices (key splits)."""
    cfg = Cfg(B=3, Hq=8, Hkv=2, D=64, C=110, W=100, seed=71, dtype=synth.BF16, kv_int8=True,
              softcap=20.0)
    syn = cfg.synth()
    vers = Versions(3)
    run = Lockstep(cfg, mode=mode, vers=vers)
    P = np.zeros(3, np.int64)
    for S, with_bias in [(150, False), (32, True), (17, False), (8, True), (48, True), (1, False)]:
        total = int((P + S).max())
        bias = _bias_nan_outside(cfg, syn, P, S, total) if with_bias else None
        run.step(P, S, bias=bias, total=total)
        P = P + S
    long = Cfg(B=1, Hq=4, Hkv=1, D=128, C=1600, W=1500, seed=72, dtype=synth.F16, kv_int8=True)
    syn = long.synth()
    vers = Versions(1)
    P0 = np.array([1700])
    K, V = seeded_cache(long, syn, P0, vers)
    run = Lockstep(long, mode=mode, K=K, V=V, vers=vers)
    P = P0.copy()
    for S in [64, 1, 40]:
        run.step(P, S)
        P = P + S
    say(f"  worst scaled error {run.worst:.3g}")


def test_int8_cache_ties_and_saturation():
    """New elements on exact ties of x / scale and far outside the code
    range: the GPU stores the oracle's codes (ties to even, saturation)."""
    cfg = Cfg(B=1, Hq=2, Hkv=1, D=16, C=8, W=8, seed=69, kv_int8=True, k_scale=0.25,
              v_scale=0.5)
    mult = np.array([2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 1.5, -1.5,
                     1000.0, -1000.0, 127.5, -128.5, 126.5, -127.5, 0.0, 7.0])
    run = Lockstep(cfg)
    q = np.random.default_rng(69).normal(size=(1, 1, 32)).astype(np.float32)
    k = (mult * 0.25).astype(np.float32).reshape(1, 1, 16)
    v = (mult * 0.5).astype(np.float32).reshape(1, 1, 16)
    run.step([0], 1, q=q, k=k, v=v)
    gk, gv = run.gpu.present_host()
    want = np.array([2, 4, -2, -4, 0, 0, 2, -2, 127, -128, 127, -128, 126, -128, 0, 7], np.int8)
    assert np.array_equal(gk[0, 0, 0], want) and np.array_equal(gv[0, 0, 0], want)


def test_int8_cache_host_errors():
    import sliding_window_gqa_02_amd as sw
    t = torch.zeros(8192, dtype=torch.float32, device="cuda:0")
    ws = torch.zeros(1 << 16, dtype=torch.int32, device="cuda:0")
    seq = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    mk = lambda **kw: sw.make_params(1, 1, 2, 2, 64, 6, 4, 8, **kw)
    assert sw.forward_status(mk(kv_cache_type=1, k_scale=0.0, v_scale=1.0), t, t, t, t, t, seq,
                             None, t, t, t, ws) == sw.ERR_ARG
    assert sw.forward_status(mk(kv_cache_type=3, k_scale=1.0, v_scale=1.0), t, t, t, t, t, seq,
                             None, t, t, t, ws) == sw.ERR_UNSUPPORTED
    p8 = sw.make_params(1, 1, 2, 2, 8, 6, 4, 8, kv_cache_type=1, k_scale=1.0, v_scale=1.0)
    assert sw.forward_status(p8, t, t, t, t, t, seq, None, t, t, t, ws) == sw.ERR_UNSUPPORTED
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# fp8 E4M3 cache (kv_cache_type 2): the int8 paths with E4M3 codes (nearest,
# ties to the even code, saturated at 448), decode and multi-token steps.
F8 = [
    Cfg(B=2, Hq=8, Hkv=2, D=64, C=40, W=33, seed=81, kv_fp8=True, k_scale=0.02, v_scale=0.03),
    Cfg(B=2, Hq=16, Hkv=2, D=128, C=70, W=64, seed=82, dtype=synth.BF16, softcap=30.0,
        kv_fp8=True, k_scale=0.01, v_scale=0.01),
    Cfg(B=1, Hq=4, Hkv=4, D=256, C=20, W=17, seed=83, dtype=synth.F16, kv_fp8=True,
        sink_std=1.0),
    Cfg(B=3, Hq=4, Hkv=2, D=32, C=30, W=20, seed=84, dtype=synth.F16, kv_fp8=True, rotary=1),
]


@pytest.mark.parametrize("mode", ["shared", "separate"])
@pytest.mark.parametrize("cfg", F8, ids=lambda c: f"D{c.D}t{c.dtype}g{c.Hq // c.Hkv}rot{c.rotary}")
def test_fp8_cache_random_steps(cfg, mode):
    say(f"fp8 cache {cfg} mode={mode}")
    rng = np.random.default_rng(cfg.seed)
    run = Lockstep(cfg, mode=mode)
    T = 0
    for _ in range(14):
        S = int(rng.choice([1, 1, 1, 2, 5, 15, 16, 33, int(rng.integers(1, 2 * cfg.C + 2))]))
        run.step([T] * cfg.B, S)
        T += S
    say(f"  worst scaled error {run.worst:.3g}")


def test_fp8_cache_codes_ties_saturation_and_key_splits():
    """Exact ties and far values on the GPU give the oracle's codes; then a
    long window over one slice (key splits) on seeded codes."""
    cfg = Cfg(B=1, Hq=2, Hkv=1, D=16, C=8, W=8, seed=85, kv_fp8=True, k_scale=1.0, v_scale=0.5)
    vals = np.array([1.0625, 1.1875, -1.0625, 2.0 ** -10, 3 * 2.0 ** -11, 7.5 * 2.0 ** -9,
                     1000.0, -1000.0, 432.0, 440.0, 447.0, -0.0, 0.3, 15.5 * 2.0 ** -9, 0.0, 5.0])
    run = Lockstep(cfg)
    q = np.random.default_rng(85).normal(size=(1, 1, 32)).astype(np.float32)
    k = vals.astype(np.float32).reshape(1, 1, 16)
    v = (vals * 0.5).astype(np.float32).reshape(1, 1, 16)
    run.step([0], 1, q=q, k=k, v=v)
    gk, gv = run.gpu.present_host()
    want = np.array([oracle.quantize_e4m3(float(x), 1.0) for x in vals], np.uint8)
    assert np.array_equal(gk[0, 0, 0].view(np.uint8), want)
    assert np.array_equal(gv[0, 0, 0].view(np.uint8), want)
    long = Cfg(B=1, Hq=4, Hkv=1, D=128, C=1600, W=1500, seed=86, dtype=synth.BF16, kv_fp8=True,
               k_scale=0.02, v_scale=0.02)
    syn = long.synth()
    vers = Versions(1)
    P0 = np.array([1700])
    K, V = seeded_cache(long, syn, P0, vers)
    run = Lockstep(long, K=K, V=V, vers=vers)
    P = P0.copy()
    for S in [1, 64, 4]:
        run.step(P, S)
        P = P + S
    say(f"  worst scaled error {run.worst:.3g}")


# ---------------------------------------------------------------------------
# HIP graph replay: a run of steps captured once through the C ABI (the
# slice counters of the in-kernel compaction included) and replayed three
# times from a restored cache, with eager work between the replays; every
# replay equals the eager run byte for byte.
@pytest.mark.parametrize("cache", ["element", "int8"])
def test_graph_replay_equals_eager(cache):
    import ctypes
    import sliding_window_gqa_02_amd as sw
    from tests.gpu_backend import to_dev
    cfg = Cfg(B=2, Hq=8, Hkv=2, D=64, C=40, W=33, seed=91, kv_int8=cache == "int8")
    syn = cfg.synth()
    vers = Versions(2)
    P0 = np.array([60, 75])
    K, V = seeded_cache(cfg, syn, P0, vers)
    Kd, Vd = to_dev(K), to_dev(V)
    snap = (Kd.clone(), Vd.clone())
    n = 24
    steps = []
    for s in range(n):
        P = P0 + s
        q, k, v = step_inputs(cfg, syn, P, 1, vers)
        steps.append((to_dev(q), to_dev(k), to_dev(v), to_dev((P).astype(np.int32))))
    p = sw.make_params(2, 1, cfg.Hq, cfg.Hkv, cfg.D, cfg.C, cfg.W, int(P0.max()) + n, cfg.dtype,
                       **cfg.cache_params())
    ws = torch.zeros(sw.workspace_size(p) // 4 + 64, dtype=torch.int32, device="cuda:0")
    sw.workspace_init(ws)
    outs = [torch.empty_like(st[0]) for st in steps]

    def run(stream):
        for (q, k, v, seq), out in zip(steps, outs):
            sw.forward(p, q, k, v, Kd, Vd, seq, None, out, Kd, Vd, ws, stream=stream)

    torch.cuda.synchronize()
    run(torch.cuda.current_stream())
    torch.cuda.synchronize()
    eager_out = torch.stack([o.clone() for o in outs])
    eager_K, eager_V = Kd.clone(), Vd.clone()
    assert sw.device_status(ws) == sw.OK
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    Kd.copy_(snap[0]), Vd.copy_(snap[1])
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            run(side)
    torch.cuda.synchronize()
    for rep in range(3):
        Kd.copy_(snap[0]), Vd.copy_(snap[1])
        for o in outs:
            o.fill_(0)
        junk = torch.randn(1 << 16, device="cuda:0").sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert bool(torch.equal(torch.stack(outs), eager_out)), f"replay {rep}: outputs"
        assert bool(torch.equal(Kd, eager_K)) and bool(torch.equal(Vd, eager_V)), f"replay {rep}: cache"
        assert int(ws[64:4096].abs().sum().item()) == 0, f"replay {rep}: slice counters"
    assert sw.device_status(ws) == sw.OK
    del g, junk
