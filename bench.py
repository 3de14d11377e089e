#!/usr/bin/env python3
"""Benchmark of the windowed-GQA decode step on one MI355X.

Headline workload (the pages' decode shape): B=1, 64 Q / 8 KV heads x 64,
fp32 cache, W=128, C=384; an 8192-token prompt prefilled in one step, then
decode steps of one token.  A "step" is one decode step of the whole path
(planner, split-K attention, split combine, append / block compaction);
`--steps` of them are timed (default 256, which crosses the compaction at
T=8352).  Inputs are synthetic (seeded, N(0,1)) and resident in HBM before the
timed region.  The decode loop is replayed from a HIP graph (value) and also
run eagerly with per-step HIP events (kernel time for the roofline).

Also reported: prefill times, the batched-serving decode (B=32, 32 Q / 8 KV
heads x 128, bf16, W=4096, C=4608, softcap 50, 128 steps) with its own
roofline, the small-slack decode (C=136), chunked-prefill (S=32) and verify
(S=8) steps of B=4 fp16 items with bias, a capacity sweep at the pages' shape,
and the CPU oracle timed on a bounded sample of the headline workload (all
host cores, and 8 threads as on the pages).  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, AMD published
# kernels that run each decode step of the two decode workloads (the
# library's launch planner picks them from the shapes: 2-query tiles x 4 per
# KV head and 4 waves for the pages' shape, one 4-query tile and 8 waves per
# slice for the batched serving decode)
HEADLINE_KERNEL = "attn_decode_kernel<0, 64, 2, 4, 3, false>"
SERVING_KERNEL = "attn_decode_kernel<2, 128, 4, 8, 3, false>"
SERVING_INT8_KERNEL = "attn_decode_q8_kernel<2, 128, 4, 8, 1>"
SERVING_FP8_KERNEL = "attn_decode_q8_kernel<2, 128, 4, 8, 2>"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
class Workload:
    def __init__(self, name, B, Hq, Hkv, D, C, W, dtype, scale=0.0, softcap=0.0, seed=0,
                 kv_int8=False, k_scale=0.0, v_scale=0.0, kv_fp8=False):
        self.name, self.B, self.Hq, self.Hkv, self.D = name, B, Hq, Hkv, D
        self.C, self.W, self.dtype, self.scale, self.softcap, self.seed = C, W, dtype, scale, softcap, seed
        self.e = 4 if dtype == 0 else 2
        self.kv_int8, self.kv_fp8, self.k_scale, self.v_scale = kv_int8, kv_fp8, k_scale, v_scale
        self.ce = 1 if (kv_int8 or kv_fp8) else self.e  # cache element bytes

    def cache_params(self) -> dict:
        if not (self.kv_int8 or self.kv_fp8):
            return {}
        return dict(kv_cache_type=2 if self.kv_fp8 else 1, k_scale=self.k_scale,
                    v_scale=self.v_scale)

    def step_bytes(self, T: np.ndarray, S: int, sw, bias: bool = False) -> dict:
        """Algorithmic HBM bytes of one step for items with lengths T (after
        the step): distinct K/V rows the queries read, Q read, output write,
        appended rows, rows moved by block compaction (read + write), and the
        attention_bias entries of visible keys."""
        row = self.D * self.e      # a query / output / new row
        crow = self.D * self.ce    # a cache row
        P = T - S
        n_kv = np.minimum(T, self.W + S - 1)
        # resident rows from the cache, the S new rows from key / value
        kv_read = int(np.sum(self.Hkv * 2 * ((n_kv - S) * crow + S * row)))
        qo = 2 * len(T) * S * self.Hq * row
        if bias:
            qo += int(np.sum(self.visible_keys(T, S))) * self.Hq * self.e
        La = np.array([sw.resident_length(int(t), self.C, self.W) for t in T])
        Lb = np.array([sw.resident_length(int(p), self.C, self.W) for p in P])
        shift = Lb + S - La
        kept = La - S
        append = int(np.sum(self.Hkv * 2 * np.minimum(S, La) * crow))
        moved = int(np.sum(np.where((shift > 0) & (kept > 0), self.Hkv * 2 * 2 * kept * crow, 0)))
        return {"kv_read": kv_read, "qo": qo, "append": append, "compaction": moved,
                "total": kv_read + qo + append + moved}


    def visible_keys(self, T: np.ndarray, S: int) -> np.ndarray:
        """Per item: sum over its S queries of the keys each one sees."""
        P = (np.asarray(T) - S)[:, None] + np.arange(S)[None, :]  # query positions
        return np.minimum(P + 1, self.W).sum(axis=1)

    def step_flops(self, T: np.ndarray, S: int) -> int:
        """QK^T and PV multiply-adds over the visible (query, key) pairs, x2."""
        return int(4 * self.D * self.Hq * np.sum(self.visible_keys(T, S)))


def storage_torch_dtype(torch, dtype):
    return torch.float32 if dtype == 0 else torch.int16


def to_dev(torch, a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda:0")


class DecodeLoop:
    """Device-resident loop of steps of S tokens each: inputs for every step
    staged in HBM, one C-ABI call per step with precomputed arguments."""

    def __init__(self, torch, sw, wl: Workload, P0: np.ndarray, nsteps: int, K, V,
                 S: int = 1, bias=None, total: int | None = None, rotary: int = -1):
        import synth
        self.torch, self.sw, self.wl = torch, sw, wl
        self.nsteps, self.S = nsteps, S
        syn = synth.Synth(wl.seed, wl.Hq, wl.Hkv, wl.D, wl.dtype)
        B = wl.B
        qs, ks, vs = [], [], []
        for s in range(nsteps):
            q, k, v = syn.step_inputs(P0 + s * S, S)
            qs.append(q), ks.append(k), vs.append(v)
        self.q = to_dev(torch, np.stack(qs))        # (n, B, S, Hq*D)
        self.k = to_dev(torch, np.stack(ks))
        self.v = to_dev(torch, np.stack(vs))
        self.seq = to_dev(torch, (P0[None, :] + S * np.arange(nsteps)[:, None] + S - 1)
                          .astype(np.int32))
        self.out = torch.empty_like(self.q)
        self.K, self.V = K, V
        self.bias = bias
        self.T = P0[None, :] + S * (np.arange(nsteps)[:, None] + 1)
        total = int(self.T.max()) if total is None else total
        rot = {}
        self.tables = (None, None)
        if rotary >= 0:  # cos / sin tables covering every position of the loop
            rows = int(self.T.max()) + 1
            rot = dict(do_rotary=1, rotary_interleaved=rotary, rotary_cache_rows=rows)
            self.tables = tuple(to_dev(torch, t) for t in synth.rotary_tables(rows, wl.D, wl.dtype))
        self.p = sw.make_params(B, S, wl.Hq, wl.Hkv, wl.D, wl.C, wl.W, total, wl.dtype,
                                wl.scale, wl.softcap, **rot, **wl.cache_params())
        nbytes = sw.workspace_size(self.p)
        self.ws = torch.zeros(nbytes // 4 + 64, dtype=torch.int32, device="cuda:0")
        sw.workspace_init(self.ws)
        lib = sw.load()
        self.fn = lib.swgqa_forward
        vp = ctypes.c_void_p
        bp = None if bias is None else vp(bias.data_ptr())
        cp, sp = (None, None) if self.tables[0] is None else \
            (vp(self.tables[0].data_ptr()), vp(self.tables[1].data_ptr()))
        self.args = []
        for s in range(nsteps):
            self.args.append((ctypes.byref(self.p), vp(self.q[s].data_ptr()),
                              vp(self.k[s].data_ptr()), vp(self.v[s].data_ptr()),
                              vp(K.data_ptr()), vp(V.data_ptr()), vp(self.seq[s].data_ptr()),
                              bp, None, cp, sp, None, vp(self.out[s].data_ptr()),
                              vp(K.data_ptr()),
                              vp(V.data_ptr()), vp(self.ws.data_ptr()),
                              ctypes.c_size_t(nbytes)))

    def run(self, stream, events=None):
        st = ctypes.c_void_p(stream.cuda_stream)
        fn = self.fn
        for s, a in enumerate(self.args):
            if events is not None:
                events[s][0].record(stream)
            rc = fn(*a, st)
            if events is not None:
                events[s][1].record(stream)
            if rc != 0:
                raise RuntimeError(f"swgqa_forward failed at step {s}: {self.sw.status_string(rc)}")

    def bytes_per_step(self):
        return [self.wl.step_bytes(self.T[s], self.S, self.sw, self.bias is not None)
                for s in range(self.nsteps)]

    def flops_per_step(self):
        return [self.wl.step_flops(self.T[s], self.S) for s in range(self.nsteps)]


def time_decode(torch, loop: DecodeLoop, snapshot, use_graph: bool):
    """Returns dict with eager per-step event times and graph/eager wall times."""
    K, V = loop.K, loop.V
    stream = torch.cuda.current_stream()

    def restore():
        K.copy_(snapshot[0])
        V.copy_(snapshot[1])

    res = {}
    # eager, with per-step events (kernel time of the step)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(loop.nsteps)]
    restore()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    loop.run(stream, ev)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    res["eager_s"] = t1 - t0
    res["step_ms"] = np.array([a.elapsed_time(b) for a, b in ev])
    eager_out = loop.out.clone()
    eager_K = K.clone()
    # graph: all steps captured once, replayed from the restored snapshot
    res["graph_s"] = None
    res["graph_ok"] = None
    if use_graph:
        try:
            g = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            side.wait_stream(stream)
            restore()
            torch.cuda.synchronize()
            with torch.cuda.stream(side):
                with torch.cuda.graph(g, stream=side):
                    loop.run(side)
            torch.cuda.synchronize()
            ok = True
            ev_a, ev_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            for rep in range(3):
                restore()
                loop.out.zero_()
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                ev_a.record()
                g.replay()
                ev_b.record()
                torch.cuda.synchronize()
                t1 = time.perf_counter()
                ok = ok and bool(torch.equal(loop.out, eager_out)) and bool(torch.equal(K, eager_K))
            res["graph_s"] = t1 - t0
            res["graph_ok"] = ok
            # one kernel per step: the replay's GPU time over the steps is the
            # kernel's average duration
            res["graph_kernel_ms"] = ev_a.elapsed_time(ev_b) / loop.nsteps
            del g
        except Exception as exc:  # report, fall back to the eager number
            res["graph_error"] = repr(exc)
    return res


# ---------------------------------------------------------------------------
def seeded_cache(torch, sw, wl: Workload, P0: np.ndarray):
    """Caches holding the contract layout for past lengths P0 (rows
    [0, L(P_b)) = regenerated positions P_b - L + r); the layout depends only
    on the length, so this equals the state a prefill + decodes would leave."""
    import synth
    shape = (wl.B, wl.Hkv, wl.C, wl.D)
    if wl.kv_int8 or wl.kv_fp8:
        # seeded codes: int8 uniform in [-100, 100]; fp8 E4M3 with random sign,
        # exponent field 0..9 and mantissa (finite values up to 7.5)
        g = torch.Generator(device="cuda:0")
        g.manual_seed(wl.seed)
        if wl.kv_int8:
            K = torch.randint(-100, 101, shape, dtype=torch.int8, device="cuda:0", generator=g)
            V = torch.randint(-100, 101, shape, dtype=torch.int8, device="cuda:0", generator=g)
        else:
            def codes():
                c = (torch.randint(0, 2, shape, device="cuda:0", generator=g) << 7) | \
                    (torch.randint(0, 10, shape, device="cuda:0", generator=g) << 3) | \
                    torch.randint(0, 8, shape, device="cuda:0", generator=g)
                return c.to(torch.uint8).view(torch.int8)
            K, V = codes(), codes()
        return K, V
    syn = synth.Synth(wl.seed, wl.Hq, wl.Hkv, wl.D, wl.dtype)
    st = storage_torch_dtype(torch, wl.dtype)
    K = torch.zeros(shape, dtype=st, device="cuda:0")
    V = torch.zeros(shape, dtype=st, device="cuda:0")
    for b, P in enumerate(P0):
        L = sw.resident_length(int(P), wl.C, wl.W)
        pos = np.arange(P - L, P)[None, :]
        heads = np.arange(wl.Hkv)[:, None]
        K[b, :, :L] = to_dev(torch, syn.kv_rows(synth.K, b, heads, pos))
        V[b, :, :L] = to_dev(torch, syn.kv_rows(synth.V, b, heads, pos))
    return K, V


def source_digest() -> str:
    """sha256 over the HIP sources, to tell whether stored counter readings
    still describe the kernels being run."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sliding_window_gqa_02_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".hpp")):
            h.update(name.encode())
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def stored_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    readings (profiles/traffic.json), or None if absent or taken from other
    kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    if data.get("source_digest") != source_digest():
        return None
    entry = data.get("kernels", {}).get(kernel)
    return None if entry is None else entry.get("hbm_bytes_per_launch")


def roofline(bytes_list, kernel_ms, kernel_name):
    """Achieved = algorithmic bytes per launch / the kernel's average
    duration (one kernel per decode step)."""
    algo = float(sum(b["total"] for b in bytes_list))
    per_launch = algo / len(bytes_list)
    achieved = per_launch / (kernel_ms / 1e3) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBPS,
            "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 5),
            "traffic": stored_traffic(kernel_name),
            "kernel": kernel_name,
            "algorithmic_bytes_per_launch": int(per_launch),
            "avg_launch_us": round(kernel_ms * 1e3, 3)}


def prefill_times(torch, sw, wl: Workload, prompts):
    import synth
    syn = synth.Synth(wl.seed, wl.Hq, wl.Hkv, wl.D, wl.dtype)
    out = {}
    shape = (wl.B, wl.Hkv, wl.C, wl.D)
    st = storage_torch_dtype(torch, wl.dtype)
    K = torch.zeros(shape, dtype=st, device="cuda:0")
    V = torch.zeros(shape, dtype=st, device="cuda:0")
    for S in prompts:
        q, k, v = syn.step_inputs(np.zeros(wl.B, np.int64), S)
        dq, dk, dv = to_dev(torch, q), to_dev(torch, k), to_dev(torch, v)
        seq = to_dev(torch, np.full(wl.B, S - 1, np.int32))
        p = sw.make_params(wl.B, S, wl.Hq, wl.Hkv, wl.D, wl.C, wl.W, S, wl.dtype, wl.scale, wl.softcap)
        ws = torch.zeros(sw.workspace_size(p) // 4 + 64, dtype=torch.int32, device="cuda:0")
        sw.workspace_init(ws)
        o = torch.empty_like(dq)
        times = []
        for _ in range(3):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            sw.forward(p, dq, dk, dv, K, V, seq, None, o, K, V, ws)
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        out[str(S)] = round(min(times[1:]), 4)
        del dq, dk, dv, o, ws
    return out, (K, V)


def copy_reference(torch, mib: int):
    """A plain device-to-device copy of `mib` MiB (read + write), timed with
    HIP events: the HBM rate a simple streaming kernel reaches on this GPU,
    and the known-size kernel that scales the traffic counters."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    best = None
    for _ in range(6):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        torch.mul(src, 1.0, out=dst)  # an elementwise streaming kernel (not a DMA copy)
        b.record()
        torch.cuda.synchronize()
        t = a.elapsed_time(b)
        best = t if best is None else min(best, t)
    bytes_moved = 2 * n * 4
    del src, dst
    return {"bytes": bytes_moved, "ms": round(best, 4),
            "GBps": round(bytes_moved / (best / 1e3) / 1e9, 1)}


def cpu_baseline(wl: Workload, P: int, max_steps: int, seconds: float, threads: int = 0):
    """The oracle (fp64, OpenMP over (item, head)) on decode steps of the
    headline workload, from a cache holding the contract layout at length P."""
    import oracle
    import synth
    from tests.scenario import Cfg, OracleBackend, Versions, seeded_cache as seed_host

    cfg = Cfg(B=wl.B, Hq=wl.Hq, Hkv=wl.Hkv, D=wl.D, C=wl.C, W=wl.W, dtype=wl.dtype,
              scale=wl.scale, softcap=wl.softcap, seed=wl.seed)
    syn = cfg.synth()
    vers = Versions(wl.B, n=P + max_steps + 8)
    K, V = seed_host(cfg, syn, [P] * wl.B, vers)
    be = OracleBackend(cfg, K, V)
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    threads = oracle.set_threads(threads if threads > 0 else cores)
    n = 0
    t_used = 0.0
    while n < max_steps and t_used < seconds:
        q, k, v = syn.step_inputs(np.full(wl.B, P + n), 1)
        t0 = time.perf_counter()
        st, _, _ = be.step(1, np.full(wl.B, P + n, np.int32), q, k, v)
        t_used += time.perf_counter() - t0
        assert st == 0
        n += 1
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(wl.B * n / t_used, 2), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{n} decode steps T={P + 1}..{P + n} of the headline workload from a "
                      f"cache holding the contract layout, fp64 oracle, {threads} OpenMP threads "
                      f"on {cpu} ({platform.machine()}), {t_used:.1f} s of CPU time",
            "ms_per_step": round(t_used / n * 1e3, 3)}


def loop_stats(torch, loop: DecodeLoop, snap, tokens_per_step: int):
    """Graph-replayed step time and throughput of a step loop, plus the eager
    per-step event times split by whether the step compacted."""
    r = time_decode(torch, loop, snap, True)
    graph = bool(r.get("graph_ok") and r["graph_s"])
    step_ms = r["graph_kernel_ms"] if graph else float(np.mean(r["step_ms"]))
    wall = r["graph_s"] if graph else r["eager_s"]
    byts = loop.bytes_per_step()
    compacting = np.array([b["compaction"] > 0 for b in byts])
    eager_us = r["step_ms"] * 1e3
    out = {"mode": "hip_graph" if graph else "eager",
           "tokens_per_s": round(tokens_per_step * loop.nsteps / wall, 1),
           "step_us": round(step_ms * 1e3, 3),
           "steps": loop.nsteps,
           "compacting_steps": int(compacting.sum()),
           "eager_step_us_p50": round(float(np.median(eager_us)), 3)}
    if compacting.any() and (~compacting).any():
        out["eager_step_us_p50_compacting"] = round(float(np.median(eager_us[compacting])), 3)
        out["eager_step_us_p50_drifting"] = round(float(np.median(eager_us[~compacting])), 3)
    total = sum(b["total"] for b in byts) / loop.nsteps
    kv = sum(b["kv_read"] for b in byts) / loop.nsteps
    moved = sum(b["compaction"] for b in byts) / loop.nsteps
    out["hbm"] = {"algorithmic_bytes_per_step": int(total), "kv_read_bytes_per_step": int(kv),
                  "compaction_bytes_per_step": int(moved),
                  "achieved_GBps": round(total / (step_ms / 1e3) / 1e9, 2),
                  "frac_of_peak": round(total / (step_ms / 1e3) / 1e9 / PEAK_HBM_GBPS, 5)}
    return out, step_ms


def small_slack(torch, sw):
    """B=1, 64 Q / 8 KV heads x 64, fp32, W=128, C=136 (G=9): 400 decode
    steps after a 512-token prompt, a block compaction every 9 steps."""
    wl = Workload("small_slack", B=1, Hq=64, Hkv=8, D=64, C=136, W=128, dtype=0,
                  scale=0.125, seed=1003)
    P0 = np.array([512])
    K, V = seeded_cache(torch, sw, wl, P0)
    snap = (K.clone(), V.clone())
    loop = DecodeLoop(torch, sw, wl, P0, 400, K, V)
    loop.run(torch.cuda.current_stream())
    torch.cuda.synchronize()
    out, _ = loop_stats(torch, loop, snap, 1)
    out["workload"] = ("decode after a 512-token prompt, B=1, 64 Q / 8 KV heads x 64, fp32, "
                       "W=128, C=136 (G=9), 400 steps")
    return out


def serving_int8(torch, sw, no_graph: bool, fp8: bool = False):
    """The batched-serving decode with an 8-bit cache (int8, or fp8 E4M3 with
    fp8=True; per-tensor scales): the same shape, half the cache bytes of
    bf16."""
    srv = Workload("batched_serving_fp8" if fp8 else "batched_serving_int8", B=32, Hq=32, Hkv=8,
                   D=128, C=4608, W=4096, dtype=2, softcap=50.0, seed=1006, kv_int8=not fp8,
                   kv_fp8=fp8, k_scale=0.02, v_scale=0.02)
    rng = np.random.default_rng(1005)
    Ps = rng.integers(4096, 32769, size=32)
    K, V = seeded_cache(torch, sw, srv, Ps)
    snap = (K.clone(), V.clone())
    loop = DecodeLoop(torch, sw, srv, Ps, 128, K, V)
    loop.run(torch.cuda.current_stream())  # warm-up
    torch.cuda.synchronize()
    r = time_decode(torch, loop, snap, not no_graph)
    byts = loop.bytes_per_step()
    graph = bool(r.get("graph_ok") and r["graph_s"])
    wall = r["graph_s"] if graph else r["eager_s"]
    kms = r["graph_kernel_ms"] if graph else float(np.mean(r["step_ms"]))
    kv = sum(b["kv_read"] for b in byts) / 128 / (kms / 1e3) / 1e9
    out = {
        "workload": f"B=32 decode, 32 Q / 8 KV heads x 128, bf16 queries, "
                    f"{'fp8 E4M3' if fp8 else 'int8'} cache "
                    "(k_scale = v_scale = 0.02), W=4096, C=4608, softcap 50, past lengths "
                    "U[4096, 32768], 128 steps",
        "tokens_per_s": round(32 * 128 / wall, 1),
        "ms_per_step": round(wall / 128 * 1e3, 5),
        "mode": "hip_graph" if graph else "eager",
        "kv_read_GBps": round(kv, 1),
        "roofline": roofline(byts, kms, SERVING_FP8_KERNEL if fp8 else SERVING_INT8_KERNEL),
    }
    del K, V, snap, loop
    return out


def rotary_decode(torch, sw, prompt: int, steps: int):
    """The headline decode with rotary embedding of the query and new key
    rows (half-split pairs, default positions): what the rotary pass adds to
    a step."""
    wl = Workload("pages_decode_rotary", B=1, Hq=64, Hkv=8, D=64, C=384, W=128, dtype=0,
                  scale=0.125, seed=1002)
    P0 = np.array([prompt])
    K, V = seeded_cache(torch, sw, wl, P0)
    snap = (K.clone(), V.clone())
    loop = DecodeLoop(torch, sw, wl, P0, steps, K, V, rotary=0)
    loop.run(torch.cuda.current_stream())
    torch.cuda.synchronize()
    out, _ = loop_stats(torch, loop, snap, 1)
    out["workload"] = (f"decode after a {prompt}-token prompt, B=1, 64 Q / 8 KV heads x 64, "
                       f"fp32, W=128, C=384, rotary on query and new keys, {steps} steps")
    return out


def capacity_sweep(torch, sw, slacks=(0, 4, 16, 32, 128, 256, 384), steps=800):
    """Decode step time against capacity at the pages' shape (W=128): the
    cache at T=2048 (as a 2048-token prefill leaves it), then `steps` decode
    steps, for C = W + slack."""
    out = []
    for slack in slacks:
        C = 128 + slack
        wl = Workload(f"sweep_c{C}", B=1, Hq=64, Hkv=8, D=64, C=C, W=128, dtype=0, scale=0.125,
                      seed=1002)
        P0 = np.array([2048])
        K, V = seeded_cache(torch, sw, wl, P0)
        snap = (K.clone(), V.clone())
        loop = DecodeLoop(torch, sw, wl, P0, steps, K, V)
        loop.run(torch.cuda.current_stream())
        torch.cuda.synchronize()
        st, _ = loop_stats(torch, loop, snap, 1)
        out.append({"capacity": C, "gap": C - 128 + 1, "step_us": st["step_us"],
                    "compacting_steps": st["compacting_steps"],
                    "eager_step_us_p50": st["eager_step_us_p50"]})
        del loop, K, V, snap
    return out


def chunked_and_verify(torch, sw):
    """B=4, 32 Q / 8 KV heads x 128, fp16, W=1024, C=1032, fp16 attention_bias
    N(0, 0.1) of width total_sequence_length: 32-token prompt chunks on items
    whose past lengths are uniform in [1024, 4096] (multi-token steps on the
    matrix cores), then verify steps of 8 draft tokens."""
    import synth
    wl = Workload("chunked_verify", B=4, Hq=32, Hkv=8, D=128, C=1032, W=1024, dtype=1,
                  seed=1004)
    rng = np.random.default_rng(1004)
    P0 = rng.integers(1024, 4097, size=4)
    nchunk, nverify = 32, 64
    total = int(P0.max()) + 32 * nchunk + 8 * nverify + 8
    syn = synth.Synth(wl.seed, wl.Hq, wl.Hkv, wl.D, wl.dtype)
    res = []
    for S, nsteps, start in ((32, nchunk, P0), (8, nverify, P0 + 32 * nchunk)):
        bias = to_dev(torch, synth.to_storage(
            syn.bias_f32(np.arange(4), np.zeros(4, np.int64), S, total), wl.dtype))
        K, V = seeded_cache(torch, sw, wl, start)
        snap = (K.clone(), V.clone())
        loop = DecodeLoop(torch, sw, wl, start, nsteps, K, V, S=S, bias=bias, total=total)
        loop.run(torch.cuda.current_stream())
        torch.cuda.synchronize()
        out, step_ms = loop_stats(torch, loop, snap, 4 * S)
        flops = float(np.mean(loop.flops_per_step()))
        peak = 2500.0  # dense fp16 MFMA, TFLOP/s
        out["mfma"] = {"achieved_TFLOPs": round(flops / (step_ms / 1e3) / 1e12, 3),
                       "peak_TFLOPs": peak,
                       "frac": round(flops / (step_ms / 1e3) / 1e12 / peak, 5),
                       "flops_per_step": int(flops)}
        out["workload"] = (f"B=4 steps of {S} tokens, 32 Q / 8 KV heads x 128, fp16 cache, "
                           f"W=1024, C=1032, fp16 bias, past lengths U[1024, 4096]"
                           + (", all drafts accepted" if S == 8 else ""))
        res.append(out)
        del loop, K, V, snap, bias
    return res[0], res[1]


# ---------------------------------------------------------------------------
def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--prompt", type=int, default=8192)
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-serving", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-mib", type=int, default=512)
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the small-slack, chunked-prefill and verify workloads")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the windowed GQA step needs no exchange "
              "between GPUs and this build runs on a single MI355X; use --gpus 1.",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    import sliding_window_gqa_02_amd as sw
    sw.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.init()

    headline = Workload("pages_decode_w128_c384", B=1, Hq=64, Hkv=8, D=64, C=384, W=128,
                        dtype=0, scale=0.125, seed=1002)
    result = {}

    # prefill (also leaves the cache at T = prompt, used by the decode loop)
    prefill = {}
    if not args.no_prefill:
        log("prefill ...")
        prompts = sorted({512, 2048, args.prompt})
        prefill, _ = prefill_times(torch, sw, headline, prompts)
        log(f"  prefill ms {prefill}")

    P0 = np.array([args.prompt])
    K, V = seeded_cache(torch, sw, headline, P0)
    snap = (K.clone(), V.clone())
    nsteps = max(args.steps, 1)
    loop = DecodeLoop(torch, sw, headline, P0, nsteps, K, V)
    # warm-up: W steps from the snapshot (the loop restores it before timing)
    warm = DecodeLoop(torch, sw, headline, P0, max(args.warmup, 1), K, V) if args.warmup else None
    if warm is not None:
        K.copy_(snap[0]), V.copy_(snap[1])
        warm.run(torch.cuda.current_stream())
        torch.cuda.synchronize()
    log("decode ...")
    r = time_decode(torch, loop, snap, not args.no_graph)
    bytes_list = loop.bytes_per_step()
    graph = bool(r.get("graph_ok") and r["graph_s"])
    wall_s = r["graph_s"] if graph else r["eager_s"]
    mode = "hip_graph" if graph else "eager"
    K_steps = nsteps
    value = headline.B * K_steps / wall_s
    step_us = r["step_ms"] * 1e3
    kernel_ms = r["graph_kernel_ms"] if graph else float(np.mean(r["step_ms"]))
    rl = roofline(bytes_list, kernel_ms, HEADLINE_KERNEL)
    kv_gbps = sum(b["kv_read"] for b in bytes_list) / K_steps / (kernel_ms / 1e3) / 1e9

    result = {
        "metric": "decode tokens/s + KV-read HBM GB/s (% peak), windowed GQA W=128 C=384",
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_s / K_steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"decode after a {args.prompt}-token prompt, B=1, 64 Q / 8 KV heads "
                               f"x 64, fp32 cache, W=128, C=384 (pages' decode shape)",
                   "global_batch": 1, "seq_len": args.prompt, "capacity": 384, "window": 128},
        "roofline": rl,
        "timing": {"mode": mode, "eager_tokens_per_s": round(headline.B * K_steps / r["eager_s"], 2),
                   "graph_ok": r.get("graph_ok"), "graph_error": r.get("graph_error"),
                   "kernel_us_avg": round(kernel_ms * 1e3, 3),
                   "eager_step_us_p10": round(float(np.percentile(step_us, 10)), 3),
                   "eager_step_us_p50": round(float(np.percentile(step_us, 50)), 3),
                   "eager_step_us_p90": round(float(np.percentile(step_us, 90)), 3),
                   "kv_read_GBps": round(kv_gbps, 2),
                   "kv_read_frac_of_peak": round(kv_gbps / PEAK_HBM_GBPS, 5)},
        "prefill_ms": prefill,
        "pages_cpu_reference": {"decode_p10_ms_prompt_8192": 0.155,
                                "hardware": "AMD EPYC 7V12, 8 intra-op threads (context only)"},
    }

    if not args.no_serving:
        log("serving decode ...")
        srv = Workload("batched_serving", B=32, Hq=32, Hkv=8, D=128, C=4608, W=4096, dtype=2,
                       softcap=50.0, seed=1005)
        rng = np.random.default_rng(1005)
        Ps = rng.integers(4096, 32769, size=32)
        Ks, Vs = seeded_cache(torch, sw, srv, Ps)
        ssnap = (Ks.clone(), Vs.clone())
        sloop = DecodeLoop(torch, sw, srv, Ps, 128, Ks, Vs)
        sloop.run(torch.cuda.current_stream())  # warm-up
        torch.cuda.synchronize()
        sr = time_decode(torch, sloop, ssnap, not args.no_graph)
        sbytes = sloop.bytes_per_step()
        sgraph = bool(sr.get("graph_ok") and sr["graph_s"])
        swall = sr["graph_s"] if sgraph else sr["eager_s"]
        skms = sr["graph_kernel_ms"] if sgraph else float(np.mean(sr["step_ms"]))
        srl = roofline(sbytes, skms, SERVING_KERNEL)
        skv = sum(b["kv_read"] for b in sbytes) / 128 / (skms / 1e3) / 1e9
        result["serving"] = {
            "workload": "B=32 decode, 32 Q / 8 KV heads x 128, bf16 cache, W=4096, C=4608, "
                        "softcap 50, past lengths U[4096, 32768], 128 steps",
            "tokens_per_s": round(32 * 128 / swall, 1),
            "ms_per_step": round(swall / 128 * 1e3, 5),
            "mode": "hip_graph" if sgraph else "eager",
            "kv_read_GBps": round(skv, 1),
            "roofline": srl,
        }
        del Ks, Vs, ssnap, sloop

    if not args.no_serving:
        log("serving decode, int8 cache ...")
        result["serving_int8"] = serving_int8(torch, sw, args.no_graph)
        log("serving decode, fp8 cache ...")
        result["serving_fp8"] = serving_int8(torch, sw, args.no_graph, fp8=True)

    if not args.no_extra:
        log("rotary decode ...")
        result["rotary_decode"] = rotary_decode(torch, sw, args.prompt, nsteps)
        log("small-slack decode ...")
        result["small_slack"] = small_slack(torch, sw)
        log("chunked prefill and verify ...")
        result["chunked_prefill"], result["verify"] = chunked_and_verify(torch, sw)
        log("capacity sweep ...")
        result["capacity_sweep"] = {
            "workload": "pages' shape (B=1, 64 Q / 8 KV heads x 64, fp32, W=128), cache at "
                        "T=2048, 800 decode steps, C = W + slack",
            "points": capacity_sweep(torch, sw)}

    result["copy_reference"] = copy_reference(torch, args.copy_mib)

    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(headline, args.prompt, 400_000, args.cpu_seconds)
        # and at the pages' 8 intra-op threads, for comparison with their figure
        result["cpu_baseline_8_threads"] = cpu_baseline(headline, args.prompt, 400_000,
                                                        args.cpu_seconds / 2, threads=8)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
