"""GPU parity at the workloads' full sizes.

The HIP path runs every step of each workload exactly as the benchmark does
(shared buffer, in place).  After every step the resident rows of the items
checked are compared byte for byte with the layout the contract fixes
(regenerated from absolute positions).  Outputs are compared with the CPU
oracle on sampled (step, item) pairs: the oracle gets the same inputs and a
past cache regenerated from positions -- never state produced by the GPU --
which is exact because the layout depends only on the length ("Specify
GroupQueryAttention windowed KV cache layout contract", Description).
The pages' decode shape and the batched serving decode are compared at
every output of every step.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from tests.parity import assert_outputs_close, say
from tests.scenario import Cfg, Versions, layout_rows, step_inputs

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sliding_window_gqa_02_amd as sw
    sw.load()


class Device:
    """Device caches of a workload, stepped through the C ABI."""

    def __init__(self, cfg: Cfg, B: int):
        import sliding_window_gqa_02_amd as sw
        from tests.gpu_backend import nan_value, torch_storage
        self.sw = sw
        self.cfg = cfg
        self.B = B
        st = torch_storage(cfg.dtype)
        self.K = torch.full((B, cfg.Hkv, cfg.C, cfg.D), nan_value(cfg.dtype), dtype=st, device="cuda:0")
        self.V = torch.full_like(self.K, nan_value(cfg.dtype))
        self.ws = None
        self.ws_bytes = 0

    def seed(self, syn, Ps, vers):
        from tests.gpu_backend import to_dev
        for b, P in enumerate(Ps):
            L, k, v = layout_rows(self.cfg, syn, b, int(P), vers)
            self.K[b, :, :L] = to_dev(k)
            self.V[b, :, :L] = to_dev(v)

    def step(self, items, P, S, q, k, v, bias=None, total=None):
        """One step for the contiguous item range `items` (a slice)."""
        from tests.gpu_backend import to_dev, to_host
        cfg, sw = self.cfg, self.sw
        P = np.asarray(P, dtype=np.int64)
        T = P + S
        total = int(T.max()) if total is None else total
        nb = len(P)
        p = sw.make_params(nb, S, cfg.Hq, cfg.Hkv, cfg.D, cfg.C, cfg.W, total, cfg.dtype,
                           cfg.scale, cfg.softcap)
        need = sw.workspace_size(p)
        if self.ws is None or need > self.ws_bytes:
            self.ws = torch.zeros(need // 4 + 64, dtype=torch.int32, device="cuda:0")
            self.ws_bytes = need
            sw.workspace_init(self.ws)
        Kv, Vv = self.K[items], self.V[items]
        dq = to_dev(q)
        out = torch.empty_like(dq)
        sw.forward(p, dq, to_dev(k), to_dev(v), Kv, Vv, to_dev((T - 1).astype(np.int32)),
                   None if bias is None else to_dev(bias), out, Kv, Vv, self.ws)
        torch.cuda.synchronize()
        st = sw.device_status(self.ws, clear=True)
        assert st == sw.OK, f"device status {st}"
        return to_host(out, cfg.dtype)

    def check_layout(self, syn, b, T, vers, what=""):
        from tests.gpu_backend import to_host
        L, k, v = layout_rows(self.cfg, syn, b, int(T), vers)
        gk = to_host(self.K[b, :, :L], self.cfg.dtype)
        gv = to_host(self.V[b, :, :L], self.cfg.dtype)
        assert np.array_equal(np.ascontiguousarray(gk).view(np.uint8), k.view(np.uint8)), f"{what} K item {b}"
        assert np.array_equal(np.ascontiguousarray(gv).view(np.uint8), v.view(np.uint8)), f"{what} V item {b}"


def oracle_item(cfg: Cfg, syn, vers, b, P, S, q, k, v, bias=None, total=None):
    """Oracle output of item b for a step of S tokens at past length P, over
    the cache layout regenerated at length P."""
    L, kk, vv = layout_rows(cfg, syn, b, int(P), vers)
    K = np.zeros((1, cfg.Hkv, cfg.C, cfg.D), dtype=synth.storage_dtype(cfg.dtype))
    V = np.zeros_like(K)
    K[0, :, :L] = kk
    V[0, :, :L] = vv
    total = int(P + S) if total is None else total
    p = cfg.params(S, total, B=1)
    st, out, _ = oracle.forward(p, np.ascontiguousarray(q), np.ascontiguousarray(k),
                                np.ascontiguousarray(v), K, V, np.array([P + S - 1], np.int32),
                                None if bias is None else np.ascontiguousarray(bias))
    assert st == 0
    return out


# ---------------------------------------------------------------------------
# The pages' decode shape: 64 Q / 8 KV heads x 64, fp32, W=128, C=384; prompts
# of 512, 2048 and 8192 tokens prefilled in one step, then 256 decode steps.
@pytest.mark.parametrize("prompt", [512, 2048, 8192])
def test_pages_shape_full(prompt):
    cfg = Cfg(B=1, Hq=64, Hkv=8, D=64, C=384, W=128, seed=1002, scale=0.125)
    syn = cfg.synth()
    vers = Versions(1, n=prompt + 300)
    dev = Device(cfg, 1)
    say(f"pages' shape prompt {prompt}: prefill")
    q, k, v = step_inputs(cfg, syn, np.array([0]), prompt, vers)
    out = dev.step(slice(0, 1), [0], prompt, q, k, v)
    dev.check_layout(syn, 0, prompt, vers, "prefill")
    # every output of the prefill
    ref = oracle_item(cfg, syn, vers, 0, 0, prompt, q, k, v)
    assert_outputs_close(out, ref, cfg.dtype, f"prefill {prompt}")
    say("  decode 256 steps")
    for s in range(256):
        P = prompt + s
        q, k, v = step_inputs(cfg, syn, np.array([P]), 1, vers)
        out = dev.step(slice(0, 1), [P], 1, q, k, v)
        dev.check_layout(syn, 0, P + 1, vers, f"decode T={P + 1}")
        ref = oracle_item(cfg, syn, vers, 0, P, 1, q, k, v)
        assert_outputs_close(out, ref, cfg.dtype, f"decode T={P + 1}")


# ---------------------------------------------------------------------------
# Chunked prefill + speculative decode: B=4, 32 Q / 8 KV heads x 128, fp16,
# W=1024, C = W+8 and W+31; prompt lengths 32 * U{32..128}; per-item 32-token
# chunks, then batched 32-token steps at ragged lengths, then batched verify
# steps of 8 drafts with k ~ U{0..7} rejected (no cache edit when exact,
# otherwise restore the item and append the accepted tokens alone);
# attention_bias fp16 ~ N(0, 0.1) in absolute key columns.
@pytest.mark.parametrize("C", [1032, 1055])
def test_chunked_prefill_speculative_full(C):
    cfg = Cfg(B=4, Hq=32, Hkv=8, D=128, C=C, W=1024, seed=1004, dtype=synth.F16)
    syn = cfg.synth()
    rng = np.random.default_rng(1004)
    n = 32 * rng.integers(32, 129, size=4)
    vers = Versions(4, n=int(n.max()) + 600)
    dev = Device(cfg, 4)

    def bias_for(items, P, S, total):
        return synth.to_storage(syn.bias_f32(items, P, S, total,
                                             version_of=lambda bi, qpos: vers.of(items[bi], qpos)),
                                cfg.dtype)

    def inputs(items, P, S):
        qs, ks, vs = [], [], []
        for bi, b in enumerate(items):
            ver = vers.of(b, P[bi] + np.arange(S))[None, :]
            pos = (P[bi] + np.arange(S))[None, :, None]
            qs.append(syn.q_rows(b, np.arange(cfg.Hq)[None, None, :], pos, ver[:, :, None]).reshape(S, -1))
            ks.append(syn.kv_rows(synth.K, b, np.arange(cfg.Hkv)[None, None, :], pos, ver[:, :, None]).reshape(S, -1))
            vs.append(syn.kv_rows(synth.V, b, np.arange(cfg.Hkv)[None, None, :], pos, ver[:, :, None]).reshape(S, -1))
        return np.stack(qs), np.stack(ks), np.stack(vs)

    T = np.zeros(4, dtype=np.int64)
    # Phase A: per-item chunked prefill of the first n_b - 256 tokens.
    say(f"C={C} phase A, prompts {list(n)}")
    checked = 0
    for b in range(4):
        nchunks = int((n[b] - 256) // 32)
        for c in range(nchunks):
            P = np.array([T[b]])
            q, k, v = inputs([b], P, 32)
            bias = bias_for([b], P, 32, int(P[0]) + 32)
            out = dev.step(slice(b, b + 1), P, 32, q, k, v, bias)
            T[b] += 32
            if c % 8 == 0 or c == nchunks - 1:
                dev.check_layout(syn, b, T[b], vers, f"A item {b} chunk {c}")
            if c in (0, 1) or c % 24 == 5 or c == nchunks - 1:
                ref = oracle_item(cfg, syn, vers, b, int(P[0]), 32, q, k, v, bias)
                assert_outputs_close(out, ref, cfg.dtype, f"A item {b} chunk {c}")
                checked += 1
    # Phase B: 8 batched 32-token steps at ragged lengths.
    say("  phase B")
    items = [0, 1, 2, 3]
    for s in range(8):
        P = T.copy()
        total = int((P + 32).max())
        q, k, v = inputs(items, P, 32)
        bias = bias_for(items, P, 32, total)
        out = dev.step(slice(0, 4), P, 32, q, k, v, bias, total)
        T += 32
        for b in range(4):
            dev.check_layout(syn, b, T[b], vers, f"B step {s}")
        b = s % 4
        ref = oracle_item(cfg, syn, vers, b, int(P[b]), 32, q[b:b + 1], k[b:b + 1], v[b:b + 1],
                          bias[b:b + 1], total)
        assert_outputs_close(out[b:b + 1], ref, cfg.dtype, f"B step {s} item {b}")
    # Phase C: 32 batched verify steps of 8 drafts.
    say("  phase C")
    exact = inexact = 0
    for s in range(32):
        P = T.copy()
        total = int((P + 8).max())
        q, k, v = inputs(items, P, 8)
        bias = bias_for(items, P, 8, total)
        snap_k, snap_v = dev.K.clone(), dev.V.clone()
        out = dev.step(slice(0, 4), P, 8, q, k, v, bias, total)
        b = s % 4
        ref = oracle_item(cfg, syn, vers, b, int(P[b]), 8, q[b:b + 1], k[b:b + 1], v[b:b + 1],
                          bias[b:b + 1], total)
        assert_outputs_close(out[b:b + 1], ref, cfg.dtype, f"C step {s} item {b}")
        for b in range(4):
            dev.check_layout(syn, b, P[b] + 8, vers, f"C step {s}")
        kk = rng.integers(0, 8, size=4)
        for b in range(4):
            Tb = int(P[b]) + 8
            rej = np.arange(Tb - kk[b], Tb)
            if oracle.rollback_exact(Tb, int(kk[b]), C, cfg.W):
                exact += 1
                T[b] = Tb - kk[b]                    # no cache edit
                vers.bump(b, rej)
            else:
                inexact += 1
                dev.K[b].copy_(snap_k[b])            # restore the item, append accepted only
                dev.V[b].copy_(snap_v[b])
                acc = 8 - int(kk[b])
                if acc:
                    Pb = np.array([P[b]])
                    q1, k1, v1 = inputs([b], Pb, acc)
                    dev.step(slice(b, b + 1), Pb, acc, q1, k1, v1,
                             bias_for([b], Pb, acc, int(Pb[0]) + acc))
                T[b] = int(P[b]) + acc
                vers.bump(b, rej)
            dev.check_layout(syn, b, T[b], vers, f"C step {s} after rollback")
    say(f"  exact rollbacks {exact}, restored {inexact}, oracle-checked chunks {checked}")
    assert exact > 0 and inexact > 0


# ---------------------------------------------------------------------------
# Batched serving decode: B=32, 32 Q / 8 KV heads x 128, bf16, W=4096,
# C=4608, softcap 50, past lengths U[4096, 32768]; 128 decode steps from a
# cache holding the contract layout.  The oracle follows all 32 items from
# the same regenerated cache (its state never comes from the GPU): every
# output of every step is compared, compacting steps included, and every
# item's resident rows at the end, byte for byte.
def test_batched_serving_full():
    from tests.gpu_backend import to_dev, to_host
    cfg = Cfg(B=32, Hq=32, Hkv=8, D=128, C=4608, W=4096, seed=1005, dtype=synth.BF16,
              softcap=50.0)
    syn = cfg.synth()
    rng = np.random.default_rng(1005)
    P0 = rng.integers(4096, 32769, size=32)
    vers = Versions(32, n=int(P0.max()) + 200)
    dev = Device(cfg, 32)
    say("serving: seeding 32 items")
    shape = (32, cfg.Hkv, cfg.C, cfg.D)
    oK = np.zeros(shape, np.uint16)
    oV = np.zeros(shape, np.uint16)
    for b, P in enumerate(P0):
        L, k, v = layout_rows(cfg, syn, b, int(P), vers)
        oK[b, :, :L] = k
        oV[b, :, :L] = v
        dev.K[b, :, :L] = to_dev(k)
        dev.V[b, :, :L] = to_dev(v)
    T = P0.copy()
    events = 0
    compacting_steps = 0
    for s in range(128):
        P = T.copy()
        q, k, v = step_inputs(cfg, syn, P, 1, vers)
        out = dev.step(slice(0, 32), P, 1, q, k, v)
        T += 1
        st, ref, plan = oracle.forward(cfg.params(1, int(T.max()), B=32), q, k, v, oK, oV,
                                       (T - 1).astype(np.int32))
        assert st == 0
        assert_outputs_close(out, ref, cfg.dtype, f"step {s}")
        n_compact = int((plan[:, 5] > 0).sum())
        events += n_compact
        compacting_steps += int(n_compact > 0)
        if n_compact or s % 32 == 0:
            gk, gv = to_host(dev.K, cfg.dtype), to_host(dev.V, cfg.dtype)
            for b in range(32):
                La = int(plan[b, 3])
                assert np.array_equal(gk[b, :, :La], oK[b, :, :La]), f"step {s} K item {b}"
                assert np.array_equal(gv[b, :, :La], oV[b, :, :La]), f"step {s} V item {b}"
            del gk, gv
        if s % 16 == 0:
            say(f"  step {s}: {events} compaction events so far")
    say(f"  compaction events {events} on {compacting_steps} steps")
    assert events > 0
    for b in range(32):
        dev.check_layout(syn, b, T[b], vers, "final")


# ---------------------------------------------------------------------------
# The batched serving decode over an 8-bit cache (int8 / fp8 E4M3), at the
# full size and in the benchmark's launch configuration: seeded codes, 48
# decode steps; four items are followed by the oracle from the same seeded
# codes, compared at every step (outputs) and at the end (resident codes byte
# for byte).
@pytest.mark.parametrize("code", ["int8", "fp8"])
def test_batched_serving_full_8bit(code):
    from tests.gpu_backend import to_dev, to_host
    import sliding_window_gqa_02_amd as sw
    fp8 = code == "fp8"
    cfg = Cfg(B=32, Hq=32, Hkv=8, D=128, C=4608, W=4096, seed=1007, dtype=synth.BF16,
              softcap=50.0, kv_int8=not fp8, kv_fp8=fp8, k_scale=0.02, v_scale=0.02)
    syn = cfg.synth()
    rng = np.random.default_rng(1007)
    P0 = rng.integers(4096, 32769, size=32)
    shape = (32, cfg.Hkv, cfg.C, cfg.D)
    if fp8:  # finite E4M3 codes up to 7.5
        codes = lambda sh: ((rng.integers(0, 2, sh) << 7) | (rng.integers(0, 10, sh) << 3) |
                            rng.integers(0, 8, sh)).astype(np.uint8).view(np.int8)
    else:
        codes = lambda sh: rng.integers(-100, 101, sh).astype(np.int8)
    K0, V0 = codes(shape), codes(shape)
    tracked = [0, 7, 19, 31]
    oK = {b: K0[b:b + 1].copy() for b in tracked}
    oV = {b: V0[b:b + 1].copy() for b in tracked}
    K = torch.from_numpy(K0).to("cuda:0")
    V = torch.from_numpy(V0).to("cuda:0")
    del K0, V0
    T = P0.copy()
    ws = None
    for s in range(48):
        P = T.copy()
        q, k, v = syn.step_inputs(P, 1)
        p = sw.make_params(32, 1, cfg.Hq, cfg.Hkv, cfg.D, cfg.C, cfg.W, int((P + 1).max()),
                           cfg.dtype, cfg.scale, cfg.softcap, **cfg.cache_params())
        if ws is None:
            ws = torch.zeros(sw.workspace_size(p) // 4 + 64, dtype=torch.int32, device="cuda:0")
            sw.workspace_init(ws)
        dq = to_dev(q)
        out = torch.empty_like(dq)
        sw.forward(p, dq, to_dev(k), to_dev(v), K, V, to_dev(P.astype(np.int32)), None, out, K, V,
                   ws)
        torch.cuda.synchronize()
        assert sw.device_status(ws, clear=True) == sw.OK
        got = to_host(out, cfg.dtype)
        for b in tracked:
            po = cfg.params(1, int(P[b]) + 1, B=1)
            st, ref, _ = oracle.forward(po, np.ascontiguousarray(q[b:b + 1]),
                                        np.ascontiguousarray(k[b:b + 1]),
                                        np.ascontiguousarray(v[b:b + 1]), oK[b], oV[b],
                                        np.array([P[b]], np.int32))
            assert st == 0
            assert_outputs_close(got[b:b + 1], ref, cfg.dtype, f"{code} step {s} item {b}")
        T += 1
    say(f"  {code}: 48 steps, items {tracked} followed by the oracle")
    gk, gv = K.cpu().numpy(), V.cpu().numpy()
    for b in tracked:
        L = oracle.resident_length(int(T[b]), cfg.C, cfg.W)
        assert np.array_equal(gk[b, :, :L], oK[b][0, :, :L]), f"{code} K item {b}"
        assert np.array_equal(gv[b, :, :L], oV[b][0, :, :L]), f"{code} V item {b}"
