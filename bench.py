#!/usr/bin/env python3
"""Benchmark of the windowed-GQA decode step on one MI355X.

Headline workload (the pages' decode shape): B=1, 64 Q / 8 KV heads x 64,
fp32 cache, W=128, C=384, decode steps of one token after an 8192-token
prompt.  A "step" is one decode step of the whole path (planner, attention,
append / block compaction).  `--steps` steps are timed (default 257, one gap
period G = C - W + 1); the timed window is placed so that it contains the
first block compaction after the prompt (T = 8352), whatever its length.
Inputs are synthetic (seeded, N(0,1)) and resident in HBM before the timed
region.  The timed steps are captured in one HIP graph and replayed five
times, each replay from the restored cache and bracketed by
synchronisations; `value` comes from HIP events on the replay stream (median
replay), the wall-clock rate is reported beside it, and an eager run with
per-step events gives p10 / p50 / p90 and the kernel time for the roofline.

Also reported: prefill times; decode after 512-, 2048- and 8192-token
prompts; the batched-serving decode (B=32, 32 Q / 8 KV heads x 128, bf16,
W=4096, C=4608, softcap 50) with bf16, int8 and fp8 caches; rotary decode;
the small-slack decode (C=136); chunked prefill (S=32), verify steps (S=8)
and verify cycles with rejected drafts (rollback or restore + re-append) at
C = 1032 and 1055; a capacity sweep at the pages' shape; the compaction's
cost wherever some steps compact and others do not; a streaming copy for
reference; and the CPU oracle timed on a bounded sample of the headline
workload (all host cores, and 8 threads as on the pages).  Prints one JSON
line.  `--only` restricts the run to some sections (profiling runs);
`--digest-counters` turns two rocprofv3 counter runs into
profiles/traffic.json.
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
HEADLINE_KERNEL = "attn_decode_kernel<0, 64, 2, 4, 3, false, false>"
SERVING_KERNEL = "attn_decode_kernel<2, 128, 4, 8, 3, false, true>"
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


def time_decode(torch, loop: DecodeLoop, snapshot, use_graph: bool, replays: int = 5,
                min_steps: int = 257):
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
    batch = max(1, -(-min_steps // loop.nsteps))
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
            gpu_ms, wall_s = [], []
            # correctness: one replay from the restored cache equals the eager run
            restore()
            loop.out.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            ok = bool(torch.equal(loop.out, eager_out)) and bool(torch.equal(K, eager_K))
            # timing: `batch` replays back to back per measurement, so that
            # the graph's start-up latency is not charged to short loops; a
            # replay after the first repeats the same steps (same lengths,
            # hence the same reads, writes and row moves) on the cache the
            # previous one left
            for rep in range(replays):
                # each measurement starts from the restored cache and is
                # bracketed by synchronisations; HIP events on the replay
                # stream time it
                restore()
                loop.out.zero_()
                ev_a = torch.cuda.Event(enable_timing=True)
                ev_b = torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                ev_a.record(stream)
                for _ in range(batch):
                    g.replay()
                ev_b.record(stream)
                torch.cuda.synchronize()
                wall_s.append((time.perf_counter() - t0) / batch)
                gpu_ms.append(ev_a.elapsed_time(ev_b) / batch)
            # median measurement, per replay of the loop: wall time (host
            # launch and sync included) and GPU time; one kernel per step, so
            # the GPU time over the steps is the kernel's average duration,
            # gaps between nodes included
            res["graph_s"] = float(np.median(wall_s))
            res["graph_gpu_s"] = float(np.median(gpu_ms)) / 1e3
            res["graph_ok"] = ok
            res["graph_batch"] = batch
            res["graph_kernel_ms"] = float(np.median(gpu_ms)) / loop.nsteps
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


def stored_traffic(label: str, kernel: str):
    """HBM bytes per launch of `kernel` in workload `label` from the committed
    rocprofv3 counter readings (profiles/traffic.json), or None if absent or
    taken from other kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    if data.get("source_digest") != source_digest():
        return None
    entry = data.get("workloads", {}).get(label, {}).get("kernels", {}).get(kernel)
    return None if entry is None else entry.get("hbm_bytes_per_launch")


def roofline(bytes_list, kernel_ms, kernel_name, label):
    """Achieved = algorithmic bytes per launch / the kernel's average
    duration (one kernel per decode step); traffic = the counter reading of
    that kernel in workload `label`, if current."""
    algo = float(sum(b["total"] for b in bytes_list))
    per_launch = algo / len(bytes_list)
    achieved = per_launch / (kernel_ms / 1e3) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBPS,
            "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 5),
            "traffic": stored_traffic(label, kernel_name),
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
        stream = torch.cuda.current_stream()
        # REPS copies of the step captured into one HIP graph and replayed:
        # HIP events on the replay stream time the GPU work of the steps
        # (their launches included) rather than the host's time to enqueue
        # one; a prefill from P = 0 reads no cache row, so every copy repeats
        # the same step
        reps = 8
        sw.forward(p, dq, dk, dv, K, V, seq, None, o, K, V, ws)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for _ in range(reps):
                    sw.forward(p, dq, dk, dv, K, V, seq, None, o, K, V, ws, stream=side)
        torch.cuda.synchronize()
        times = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            g.replay()
            b.record(stream)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) / reps)
        out[str(S)] = round(float(np.median(times)), 4)
        del g, dq, dk, dv, o, ws
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


def loop_stats(torch, loop: DecodeLoop, snap, tokens_per_step: int, use_graph: bool = True,
               replays: int = 5):
    """Throughput of a step loop from the GPU time of its graph replay (HIP
    events on the replay stream; wall time beside it), the eager per-step
    event times (p10 / p50 / p90), and -- where some steps compact and some
    do not -- the compaction's cost: the p50 difference between compacting
    and drifting steps, and the bytes it moves over that difference."""
    r = time_decode(torch, loop, snap, use_graph, replays)
    graph = bool(r.get("graph_ok") and r["graph_s"])
    step_ms = r["graph_kernel_ms"] if graph else float(np.mean(r["step_ms"]))
    gpu_s = r["graph_gpu_s"] if graph else float(np.sum(r["step_ms"])) / 1e3
    wall = r["graph_s"] if graph else r["eager_s"]
    byts = loop.bytes_per_step()
    compacting = np.array([b["compaction"] > 0 for b in byts])
    eager_us = r["step_ms"] * 1e3
    n = loop.nsteps
    out = {"mode": "hip_graph" if graph else "eager",
           "tokens_per_s": round(tokens_per_step * n / gpu_s, 1),
           "tokens_per_s_wall": round(tokens_per_step * n / wall, 1),
           "step_us": round(step_ms * 1e3, 3),
           "steps": n,
           "compacting_steps": int(compacting.sum()),
           "eager_step_us_p10": round(float(np.percentile(eager_us, 10)), 3),
           "eager_step_us_p50": round(float(np.percentile(eager_us, 50)), 3),
           "eager_step_us_p90": round(float(np.percentile(eager_us, 90)), 3)}
    if graph:
        out["graph_replay_identical_to_eager"] = bool(r["graph_ok"])
    if compacting.any() and (~compacting).any():
        p50c = float(np.median(eager_us[compacting]))
        p50d = float(np.median(eager_us[~compacting]))
        moved = float(np.mean([b["compaction"] for b, c in zip(byts, compacting) if c]))
        extra = p50c - p50d
        comp = {"eager_step_us_p50_compacting": round(p50c, 3),
                "eager_step_us_p50_drifting": round(p50d, 3),
                "extra_us": round(extra, 3),
                "moved_bytes_per_compacting_step": int(moved)}
        if extra > 0:
            comp["effective_GBps"] = round(moved / (extra * 1e-6) / 1e9, 1)
            comp["frac_of_peak"] = round(moved / (extra * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)
        out["compaction"] = comp
    total = sum(b["total"] for b in byts) / n
    kv = sum(b["kv_read"] for b in byts) / n
    moved = sum(b["compaction"] for b in byts) / n
    out["hbm"] = {"algorithmic_bytes_per_step": int(total), "kv_read_bytes_per_step": int(kv),
                  "compaction_bytes_per_step": int(moved),
                  "achieved_GBps": round(total / (step_ms / 1e3) / 1e9, 2),
                  "frac_of_peak": round(total / (step_ms / 1e3) / 1e9 / PEAK_HBM_GBPS, 5),
                  "kv_read_GBps": round(kv / (step_ms / 1e3) / 1e9, 2)}
    return out, step_ms, r


def small_slack(torch, sw, steps: int = 400, use_graph: bool = True):
    """B=1, 64 Q / 8 KV heads x 64, fp32, W=128, C=136 (G=9): decode steps
    after a 512-token prompt, a block compaction every 9 steps."""
    wl = Workload("small_slack", B=1, Hq=64, Hkv=8, D=64, C=136, W=128, dtype=0,
                  scale=0.125, seed=1003)
    P0 = np.array([512])
    K, V = seeded_cache(torch, sw, wl, P0)
    snap = (K.clone(), V.clone())
    loop = DecodeLoop(torch, sw, wl, P0, steps, K, V)
    loop.run(torch.cuda.current_stream())
    torch.cuda.synchronize()
    out, _, _ = loop_stats(torch, loop, snap, 1, use_graph)
    out["workload"] = ("decode after a 512-token prompt, B=1, 64 Q / 8 KV heads x 64, fp32, "
                       f"W=128, C=136 (G=9), {steps} steps")
    return out


SERVING_KINDS = {
    "bf16": ("bf16 cache", SERVING_KERNEL, {}),
    "int8": ("int8 cache (k_scale = v_scale = 0.02)", SERVING_INT8_KERNEL,
             dict(kv_int8=True, k_scale=0.02, v_scale=0.02)),
    "fp8": ("fp8 E4M3 cache (k_scale = v_scale = 0.02)", SERVING_FP8_KERNEL,
            dict(kv_fp8=True, k_scale=0.02, v_scale=0.02)),
}


def serving(torch, sw, kind: str, use_graph: bool, steps: int = 128):
    """The batched-serving decode: B=32, 32 Q / 8 KV heads x 128, bf16
    queries, W=4096, C=4608, softcap 50, past lengths U[4096, 32768]; the
    cache in bf16, or as int8 / fp8 codes (half the bytes)."""
    what, kernel, extra = SERVING_KINDS[kind]
    srv = Workload(f"batched_serving_{kind}", B=32, Hq=32, Hkv=8, D=128, C=4608, W=4096,
                   dtype=2, softcap=50.0, seed=1005 if kind == "bf16" else 1006, **extra)
    rng = np.random.default_rng(1005)
    Ps = rng.integers(4096, 32769, size=32)
    K, V = seeded_cache(torch, sw, srv, Ps)
    snap = (K.clone(), V.clone())
    loop = DecodeLoop(torch, sw, srv, Ps, steps, K, V)
    loop.run(torch.cuda.current_stream())  # warm-up
    torch.cuda.synchronize()
    out, kms, r = loop_stats(torch, loop, snap, 32, use_graph)
    out["workload"] = (f"B=32 decode, 32 Q / 8 KV heads x 128, bf16 queries, {what}, W=4096, "
                       f"C=4608, softcap 50, past lengths U[4096, 32768], {steps} steps")
    out["ms_per_step"] = round(kms, 5)
    out["roofline"] = roofline(loop.bytes_per_step(), kms, kernel, "serving")
    del K, V, snap, loop
    return out


def rotary_decode(torch, sw, prompt: int, steps: int, use_graph: bool = True):
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
    out, _, _ = loop_stats(torch, loop, snap, 1, use_graph)
    out["workload"] = (f"decode after a {prompt}-token prompt, B=1, 64 Q / 8 KV heads x 64, "
                       f"fp32, W=128, C=384, rotary on query and new keys, {steps} steps")
    return out


def capacity_sweep(torch, sw, slacks=(0, 4, 16, 32, 128, 256, 384), steps=800,
                   use_graph: bool = True):
    """Decode step time against capacity at the pages' shape (W=128): the
    cache at T=2048 (as a 2048-token prefill leaves it), then `steps` decode
    steps, for C = W + slack.  At C = W every step compacts (127 rows per
    slice): its bytes over its extra time against the drifting steps of the
    widest capacity are the in-kernel compaction's rate."""
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
        st, _, _ = loop_stats(torch, loop, snap, 1, use_graph)
        pt = {"capacity": C, "gap": C - 128 + 1, "step_us": st["step_us"],
              "compacting_steps": st["compacting_steps"],
              "eager_step_us_p50": st["eager_step_us_p50"],
              "compaction_bytes_per_step": st["hbm"]["compaction_bytes_per_step"]}
        if "compaction" in st:
            pt["compaction"] = st["compaction"]
        out.append(pt)
        del loop, K, V, snap
    first, last = out[0], out[-1]
    if (len(out) > 1 and first["compacting_steps"] == steps and
            last["compacting_steps"] < steps // 10):
        extra = first["step_us"] - last["step_us"]
        moved = first["compaction_bytes_per_step"]
        res = {"extra_us_per_step_at_C_eq_W": round(extra, 3),
               "moved_bytes_per_step_at_C_eq_W": moved}
        if extra > 0:
            res["effective_GBps"] = round(moved / (extra * 1e-6) / 1e9, 1)
            res["frac_of_peak"] = round(moved / (extra * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)
        return out, res
    return out, None


def _dev_args(vp, t):
    return None if t is None else vp(t.data_ptr())


def chunked_prefill(torch, sw, C: int, nsteps: int = 32, use_graph: bool = True):
    """B=4, 32 Q / 8 KV heads x 128, fp16, W=1024, capacity C, fp16
    attention_bias N(0, 0.1) of width total_sequence_length: 32-token prompt
    chunks on items whose past lengths are uniform in [1024, 4096] (matrix-
    core steps; every step compacts, and at C = 1032 every step is staged)."""
    import synth
    wl = Workload(f"chunked_c{C}", B=4, Hq=32, Hkv=8, D=128, C=C, W=1024, dtype=1, seed=1004)
    rng = np.random.default_rng(1004)
    P0 = rng.integers(1024, 4097, size=4)
    S = 32
    total = int(P0.max()) + S * nsteps
    syn = synth.Synth(wl.seed, wl.Hq, wl.Hkv, wl.D, wl.dtype)
    bias = to_dev(torch, synth.to_storage(
        syn.bias_f32(np.arange(4), np.zeros(4, np.int64), S, total), wl.dtype))
    K, V = seeded_cache(torch, sw, wl, P0)
    snap = (K.clone(), V.clone())
    loop = DecodeLoop(torch, sw, wl, P0, nsteps, K, V, S=S, bias=bias, total=total)
    loop.run(torch.cuda.current_stream())
    torch.cuda.synchronize()
    out, step_ms, _ = loop_stats(torch, loop, snap, 4 * S, use_graph)
    flops = float(np.mean(loop.flops_per_step()))
    peak = 2500.0  # dense fp16 MFMA, TFLOP/s
    out["mfma"] = {"achieved_TFLOPs": round(flops / (step_ms / 1e3) / 1e12, 3),
                   "peak_TFLOPs": peak,
                   "frac": round(flops / (step_ms / 1e3) / 1e12 / peak, 5),
                   "flops_per_step": int(flops)}
    out["workload"] = (f"B=4 steps of {S} tokens, 32 Q / 8 KV heads x 128, fp16 cache, "
                       f"W=1024, C={C}, fp16 bias, past lengths U[1024, 4096]")
    del loop, K, V, snap, bias
    return out


def verify_with_rejection(torch, sw, C: int, nverify: int = 32, use_graph: bool = True):
    """Speculative verify cycles at B=4, 32 Q / 8 KV heads x 128, fp16,
    W=1024, capacity C, fp16 bias: each cycle is one batched step of 8 draft
    tokens per item, after which k ~ U{0..7} drafts of each item are
    rejected.  Where L(T - k) = L(T) - k the rejection needs no cache edit
    (the next step starts at T - k); otherwise the item's resident rows are
    restored from a copy taken before the step and its 8 - k accepted tokens
    are appended by a one-item step.  The whole sequence is fixed in advance
    (it depends only on the lengths), so it replays from one HIP graph."""
    import synth
    wl = Workload(f"verify_c{C}", B=4, Hq=32, Hkv=8, D=128, C=C, W=1024, dtype=1, seed=1004)
    rng = np.random.default_rng(1004)
    P0 = rng.integers(1024, 4097, size=4) + 32 * 32
    S = 8
    total = int(P0.max()) + S * nverify + 8
    syn = synth.Synth(wl.seed, wl.Hq, wl.Hkv, wl.D, wl.dtype)
    lib = sw.load()
    vp = ctypes.c_void_p
    K, V = seeded_cache(torch, sw, wl, P0)
    snap = (K.clone(), V.clone())
    saveK = torch.empty_like(K)
    saveV = torch.empty_like(V)
    p_step = sw.make_params(4, S, wl.Hq, wl.Hkv, wl.D, C, wl.W, total, wl.dtype)
    p_one = {acc: sw.make_params(1, acc, wl.Hq, wl.Hkv, wl.D, C, wl.W, total, wl.dtype)
             for acc in range(1, S)}
    ws_bytes = max(sw.workspace_size(p) for p in [p_step, *p_one.values()])
    ws = torch.zeros(ws_bytes // 4 + 64, dtype=torch.int32, device="cuda:0")
    sw.workspace_init(ws)
    krng = np.random.default_rng(2004 + C)
    T = P0.copy()
    cycles = []   # per cycle: (inputs, items to restore with their Lb, one-item appends)
    stats = {"exact": 0, "restored": 0, "accepted_tokens": 0, "draft_tokens": 0}
    bytes_method = []
    bytes_restore = []
    for c in range(nverify):
        P = T.copy()
        q, k, v = syn.step_inputs(P, S)
        dq, dk, dv = to_dev(torch, q), to_dev(torch, k), to_dev(torch, v)
        bias = to_dev(torch, synth.to_storage(syn.bias_f32(np.arange(4), P, S, total), wl.dtype))
        seq = to_dev(torch, (P + S - 1).astype(np.int32))
        out = torch.empty_like(dq)
        kk = krng.integers(0, 8, size=4)
        restores, appends = [], []
        method = wl.step_bytes(P + S, S, sw, bias=True)["total"]
        rest = 0
        for b in range(4):
            Tb = int(P[b]) + S
            acc = S - int(kk[b])
            stats["draft_tokens"] += S
            stats["accepted_tokens"] += acc
            if sw.rollback_exact(Tb, int(kk[b]), C, wl.W):
                stats["exact"] += 1
                T[b] = Tb - kk[b]
                continue
            stats["restored"] += 1
            Lb = sw.resident_length(int(P[b]), C, wl.W)
            restores.append((b, Lb))
            rest += 2 * 2 * 2 * wl.Hkv * Lb * wl.D * wl.e   # save + restore, K and V
            if acc:
                bb = bias[b:b + 1, :, :acc, :].contiguous()
                sq = to_dev(torch, np.array([int(P[b]) + acc - 1], np.int32))
                o1 = torch.empty((1, acc, wl.Hq * wl.D), dtype=dq.dtype, device="cuda:0")
                appends.append((acc, dq[b:b + 1, :acc], dk[b:b + 1, :acc], dv[b:b + 1, :acc],
                                bb, sq, o1, b))
                method += wl.step_bytes(np.array([int(P[b]) + acc]), acc, sw, bias=True)["total"]
            T[b] = int(P[b]) + acc
        bytes_method.append(method)
        bytes_restore.append(rest)
        cycles.append(((dq, dk, dv, bias, seq, out), restores, appends))
    nbytes = ctypes.c_size_t(ws.numel() * 4)

    def run(stream, events=None):
        st = ctypes.c_void_p(stream.cuda_stream)
        with torch.cuda.stream(stream):
            for ci, ((dq, dk, dv, bias, seq, out), restores, appends) in enumerate(cycles):
                if events is not None:
                    events[ci][0].record(stream)
                for b, Lb in restores:   # copies of the rows a rejection may need back
                    saveK[b, :, :Lb].copy_(K[b, :, :Lb])
                    saveV[b, :, :Lb].copy_(V[b, :, :Lb])
                rc = lib.swgqa_forward(ctypes.byref(p_step), vp(dq.data_ptr()), vp(dk.data_ptr()),
                                       vp(dv.data_ptr()), vp(K.data_ptr()), vp(V.data_ptr()),
                                       vp(seq.data_ptr()), vp(bias.data_ptr()), None, None, None,
                                       None, vp(out.data_ptr()), vp(K.data_ptr()),
                                       vp(V.data_ptr()), vp(ws.data_ptr()), nbytes, st)
                if rc != 0:
                    raise RuntimeError(f"verify step {ci}: {sw.status_string(rc)}")
                for b, Lb in restores:
                    K[b, :, :Lb].copy_(saveK[b, :, :Lb])
                    V[b, :, :Lb].copy_(saveV[b, :, :Lb])
                for acc, q1, k1, v1, b1, s1, o1, b in appends:
                    Kb, Vb = K[b:b + 1], V[b:b + 1]
                    rc = lib.swgqa_forward(ctypes.byref(p_one[acc]), vp(q1.data_ptr()),
                                           vp(k1.data_ptr()), vp(v1.data_ptr()),
                                           vp(Kb.data_ptr()), vp(Vb.data_ptr()),
                                           vp(s1.data_ptr()), vp(b1.data_ptr()), None, None,
                                           None, None, vp(o1.data_ptr()), vp(Kb.data_ptr()),
                                           vp(Vb.data_ptr()), vp(ws.data_ptr()), nbytes, st)
                    if rc != 0:
                        raise RuntimeError(f"one-item append {ci}: {sw.status_string(rc)}")
                if events is not None:
                    events[ci][1].record(stream)

    def restore():
        K.copy_(snap[0])
        V.copy_(snap[1])

    stream = torch.cuda.current_stream()
    restore()
    run(stream)   # warm-up
    torch.cuda.synchronize()
    restore()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(nverify)]
    torch.cuda.synchronize()
    run(stream, ev)
    torch.cuda.synchronize()
    eager_us = np.array([a.elapsed_time(b) for a, b in ev]) * 1e3
    eager_K = K.clone()
    res = {"mode": "eager"}
    gpu_s = float(np.sum(eager_us)) / 1e6
    if use_graph:
        try:
            g = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            restore()
            torch.cuda.synchronize()
            with torch.cuda.stream(side):
                with torch.cuda.graph(g, stream=side):
                    run(side)
            times, ok = [], True
            for rep in range(5):
                restore()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                a.record(stream)
                g.replay()
                b.record(stream)
                torch.cuda.synchronize()
                times.append(a.elapsed_time(b))
                ok = ok and bool(torch.equal(K, eager_K))
            gpu_s = float(np.median(times)) / 1e3
            res = {"mode": "hip_graph", "graph_replay_identical_to_eager": ok}
            del g
        except Exception as exc:
            res["graph_error"] = repr(exc)
    cyc_us = gpu_s / nverify * 1e6
    mb = float(np.mean(bytes_method))
    res.update({
        "workload": (f"B=4 verify cycles of 8 draft tokens, 32 Q / 8 KV heads x 128, fp16 cache, "
                     f"W=1024, C={C}, fp16 bias, k ~ U{{0..7}} drafts rejected per item: no cache "
                     f"edit when exact, else the item restored and its accepted tokens appended "
                     f"by a one-item step; {nverify} cycles"),
        "cycle_us": round(cyc_us, 3),
        "accepted_tokens_per_s": round(stats["accepted_tokens"] / gpu_s, 1),
        "draft_tokens_per_s": round(stats["draft_tokens"] / gpu_s, 1),
        "eager_cycle_us_p10": round(float(np.percentile(eager_us, 10)), 3),
        "eager_cycle_us_p50": round(float(np.percentile(eager_us, 50)), 3),
        "eager_cycle_us_p90": round(float(np.percentile(eager_us, 90)), 3),
        "rollbacks_exact": stats["exact"], "rollbacks_restored": stats["restored"],
        "hbm": {"algorithmic_bytes_per_cycle": int(mb),
                "restore_copy_bytes_per_cycle": int(np.mean(bytes_restore)),
                "achieved_GBps": round(mb / (cyc_us * 1e-6) / 1e9, 2),
                "frac_of_peak": round(mb / (cyc_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 5)},
    })
    del cycles, K, V, snap, saveK, saveV, ws
    return res


def verify_steps(torch, sw, C: int, nsteps: int = 64, use_graph: bool = True):
    """The verify step alone (B=4, 8 draft tokens per item, every draft
    accepted): one launch sequence per step, for its roofline."""
    import synth
    wl = Workload(f"verify_steps_c{C}", B=4, Hq=32, Hkv=8, D=128, C=C, W=1024, dtype=1,
                  seed=1004)
    rng = np.random.default_rng(1004)
    P0 = rng.integers(1024, 4097, size=4) + 32 * 32
    S = 8
    total = int(P0.max()) + S * nsteps
    syn = synth.Synth(wl.seed, wl.Hq, wl.Hkv, wl.D, wl.dtype)
    bias = to_dev(torch, synth.to_storage(
        syn.bias_f32(np.arange(4), np.zeros(4, np.int64), S, total), wl.dtype))
    K, V = seeded_cache(torch, sw, wl, P0)
    snap = (K.clone(), V.clone())
    loop = DecodeLoop(torch, sw, wl, P0, nsteps, K, V, S=S, bias=bias, total=total)
    loop.run(torch.cuda.current_stream())
    torch.cuda.synchronize()
    out, step_ms, _ = loop_stats(torch, loop, snap, 4 * S, use_graph)
    flops = float(np.mean(loop.flops_per_step()))
    out["mfma"] = {"achieved_TFLOPs": round(flops / (step_ms / 1e3) / 1e12, 3),
                   "peak_TFLOPs": 2500.0,
                   "frac": round(flops / (step_ms / 1e3) / 1e12 / 2500.0, 5),
                   "flops_per_step": int(flops)}
    out["workload"] = (f"B=4 steps of 8 tokens, 32 Q / 8 KV heads x 128, fp16 cache, W=1024, "
                       f"C={C}, fp16 bias, past lengths U[2048, 5120], all drafts accepted")
    del loop, K, V, snap, bias
    return out


def first_compaction_after(T0: int, C: int, W: int, sw) -> int:
    """First total length T > T0 whose one-token step compacts."""
    T = T0 + 1
    while sw.resident_length(T, C, W) == sw.resident_length(T - 1, C, W) + 1:
        T += 1
    return T


def decode_after_prompt(torch, sw, wl: Workload, prompt: int, steps: int, use_graph: bool,
                        warmup: int = 0, window_on_compaction: bool = False):
    """Decode steps of the pages' shape after a prompt of `prompt` tokens (the
    cache holds the contract layout of that length).  With
    window_on_compaction the timed window starts late enough after the
    prompt that it contains the first block compaction."""
    start = prompt
    Tc = first_compaction_after(prompt, wl.C, wl.W, sw)
    if window_on_compaction:
        start = prompt + max(0, (Tc - 1 - prompt) - steps // 2)
    P0 = np.array([start])
    K, V = seeded_cache(torch, sw, wl, P0)
    snap = (K.clone(), V.clone())
    loop = DecodeLoop(torch, sw, wl, P0, steps, K, V)
    if warmup:
        warm = DecodeLoop(torch, sw, wl, P0, warmup, K, V)
        warm.run(torch.cuda.current_stream())
        torch.cuda.synchronize()
        del warm
    out, kms, r = loop_stats(torch, loop, snap, wl.B, use_graph)
    out["first_T"] = int(start + 1)
    out["last_T"] = int(start + steps)
    out["compaction_at_T"] = int(Tc)
    return out, kms, r, loop


# ---------------------------------------------------------------------------
SECTIONS = ("prefill", "headline", "decode_prompts", "serving", "serving_int8", "serving_fp8",
            "rotary", "small_slack", "chunked", "capacity", "copy", "cpu")


def digest_counters(label: str, fetch_dir: str, write_dir: str, ref_kernel: str,
                    ref_bytes: int):
    """Adds the readings of two rocprofv3 --pmc runs (FETCH_SIZE, then
    WRITE_SIZE; csv output) of one workload to profiles/traffic.json, under
    `label`: per kernel, HBM bytes per dispatch -- each counter scaled by
    what it reads for the bench's reference streaming kernel of known size
    -- as the mean for each of this library's kernels, and, where the
    dispatches form two groups (e.g. steps that compact and steps that do
    not), the mean and count of the dispatches above and below the midpoint
    of their range."""
    import csv
    import glob

    def read(d, counter):
        rows = {}
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for row in csv.DictReader(f):
                    if row.get("Counter_Name") != counter:
                        continue
                    rows.setdefault(row["Kernel_Name"], []).append(
                        (int(row["Dispatch_Id"]), float(row["Counter_Value"])))
        return {k: [v for _, v in sorted(vs)] for k, vs in rows.items()}

    fetch = read(fetch_dir, "FETCH_SIZE")
    write = read(write_dir, "WRITE_SIZE")
    ref = [k for k in fetch if ref_kernel in k]
    if not ref or ref[0] not in write:
        raise SystemExit(f"reference kernel {ref_kernel!r} not in the counter output")

    def big(vals):
        # the reference's own dispatches: the large ones (the same functor
        # may also run on small tensors)
        v = np.array(vals)
        return float(np.median(v[v >= 0.5 * v.max()]))

    # the reference kernel reads and writes ref_bytes / 2 each
    f_scale = (ref_bytes / 2) / (big(fetch[ref[0]]) * 1024)
    w_scale = (ref_bytes / 2) / (big(write[ref[0]]) * 1024)
    kernels = {}
    for name in sorted(set(fetch) & set(write)):
        if "swgqa::" not in name:
            continue
        fv, wv = np.array(fetch[name]), np.array(write[name])
        n = min(len(fv), len(wv))
        per = fv[:n] * 1024 * f_scale + wv[:n] * 1024 * w_scale
        short = name.replace("void ", "").replace("swgqa::(anonymous namespace)::", "")
        short = short.split("(")[0]
        e = {"dispatches": int(n),
             "fetch_size_KiB_raw": round(float(fv[:n].mean()), 1),
             "write_size_KiB_raw": round(float(wv[:n].mean()), 1),
             "hbm_bytes_per_launch": int(per.mean())}
        lo, hi = float(per.min()), float(per.max())
        if n > 1 and hi > 1.2 * lo:
            mid = 0.5 * (lo + hi)
            e["high_group"] = {"dispatches": int((per > mid).sum()),
                               "hbm_bytes_per_launch": int(per[per > mid].mean())}
            e["low_group"] = {"dispatches": int((per <= mid).sum()),
                              "hbm_bytes_per_launch": int(per[per <= mid].mean())}
        kernels[short] = e
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        data = {}
    if data.get("source_digest") != source_digest():
        data = {"source_digest": source_digest(), "workloads": {}}
    data["reference_kernel"] = ref[0][:120]
    data["reference_bytes_read_and_written"] = ref_bytes
    data.setdefault("workloads", {})[label] = {"fetch_scale": round(f_scale, 4),
                                               "write_scale": round(w_scale, 4),
                                               "kernels": kernels}
    with open(path, "w") as f:
        json.dump(data, f, indent=1)
    print(f"{path}: {label}: {len(kernels)} kernels, fetch x{f_scale:.3f}, write x{w_scale:.3f}")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=257,
                    help="timed headline decode steps (default: one gap period, G = 257)")
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--prompt", type=int, default=8192)
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--only", default=",".join(SECTIONS),
                    help="comma list of sections to run: " + ",".join(SECTIONS))
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-mib", type=int, default=512)
    ap.add_argument("--chunk-capacities", default="1032,1055",
                    help="cache capacities of the chunked prefill / verify sections")
    ap.add_argument("--capacity-slacks", default="0,4,16,32,128,256,384",
                    help="C - W values of the capacity sweep")
    ap.add_argument("--digest-counters", nargs=3, metavar=("LABEL", "FETCH_DIR", "WRITE_DIR"),
                    help="add the readings of two rocprofv3 --pmc csv runs of one workload "
                         "to profiles/traffic.json")
    args = ap.parse_args()

    if args.digest_counters:
        digest_counters(args.digest_counters[0], args.digest_counters[1], args.digest_counters[2],
                        "AUnaryFunctor<float, float, float, at::native::binary_internal::MulFunctor<float>",
                        2 * args.copy_mib * (1 << 20))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the windowed GQA step needs no exchange "
              "between GPUs and this build runs on a single MI355X; use --gpus 1.",
              file=sys.stderr, flush=True)
        sys.exit(2)
    only = set(x.strip() for x in args.only.split(",") if x.strip())
    unknown = only - set(SECTIONS)
    if unknown:
        raise SystemExit(f"unknown sections {sorted(unknown)}")

    import torch
    import sliding_window_gqa_02_amd as sw
    sw.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.init()
    use_graph = not args.no_graph

    headline = Workload("pages_decode_w128_c384", B=1, Hq=64, Hkv=8, D=64, C=384, W=128,
                        dtype=0, scale=0.125, seed=1002)
    K_steps = max(args.steps, 1)
    result = {
        "metric": "decode tokens/s + KV-read HBM GB/s (% peak), windowed GQA W=128 C=384",
        "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": K_steps,
        "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"decode after a {args.prompt}-token prompt, B=1, 64 Q / 8 KV "
                               f"heads x 64, fp32 cache, W=128, C=384 (pages' decode shape)",
                   "global_batch": 1, "seq_len": args.prompt, "capacity": 384, "window": 128},
    }

    if "prefill" in only:
        log("prefill ...")
        prompts = sorted({512, 2048, args.prompt})
        result["prefill_ms"], _ = prefill_times(torch, sw, headline, prompts)
        log(f"  prefill ms {result['prefill_ms']}")

    if "headline" in only:
        log("decode (headline) ...")
        st, kernel_ms, r, loop = decode_after_prompt(
            torch, sw, headline, args.prompt, K_steps, use_graph, warmup=args.warmup,
            window_on_compaction=True)
        bytes_list = loop.bytes_per_step()
        graph = st["mode"] == "hip_graph"
        gpu_s = r["graph_gpu_s"] if graph else float(np.sum(r["step_ms"])) / 1e3
        kv_gbps = sum(b["kv_read"] for b in bytes_list) / K_steps / (kernel_ms / 1e3) / 1e9
        result.update({
            "value": round(headline.B * K_steps / gpu_s, 2),
            "ms_per_step": round(gpu_s / K_steps * 1e3, 5),
            "roofline": roofline(bytes_list, kernel_ms, HEADLINE_KERNEL, "headline"),
        })
        result["timing"] = {
            "mode": st["mode"],
            "value_basis": f"HIP events on the replay stream around {r.get('graph_batch', 1)} "
                           f"back-to-back graph replay(s) of the {K_steps} timed steps from the "
                           "restored cache, synchronised before and after; median of 5",
            "tokens_per_s_wall": st["tokens_per_s_wall"],
            "eager_tokens_per_s": round(headline.B * K_steps / r["eager_s"], 2),
            "graph_replay_identical_to_eager": st.get("graph_replay_identical_to_eager"),
            "graph_error": r.get("graph_error"),
            "kernel_us_avg": round(kernel_ms * 1e3, 3),
            "eager_step_us_p10": st["eager_step_us_p10"],
            "eager_step_us_p50": st["eager_step_us_p50"],
            "eager_step_us_p90": st["eager_step_us_p90"],
            "timed_T": [st["first_T"], st["last_T"]],
            "compaction_at_T": st["compaction_at_T"],
            "compacting_steps": st["compacting_steps"],
            "kv_read_GBps": round(kv_gbps, 2),
            "kv_read_frac_of_peak": round(kv_gbps / PEAK_HBM_GBPS, 5)}
        if "compaction" in st:
            result["timing"]["compaction"] = st["compaction"]
        result["pages_cpu_reference"] = {
            "decode_p10_ms_prompt_8192": 0.155,
            "hardware": "AMD EPYC 7V12, 8 intra-op threads (context only)"}
        del loop

    if "decode_prompts" in only:
        log("decode after each prompt ...")
        dp = {}
        for prompt in sorted({512, 2048, 8192}):
            st, _, _, loop = decode_after_prompt(torch, sw, headline, prompt, 256, use_graph)
            st["workload"] = (f"256 decode steps after a {prompt}-token prompt, pages' decode "
                              "shape (B=1, 64 Q / 8 KV heads x 64, fp32, W=128, C=384)")
            dp[str(prompt)] = st
            del loop
        result["decode_after_prompt"] = dp

    for kind in ("bf16", "int8", "fp8"):
        sec = "serving" if kind == "bf16" else f"serving_{kind}"
        if sec in only:
            log(f"serving decode, {kind} cache ...")
            result[sec] = serving(torch, sw, kind, use_graph)

    if "rotary" in only:
        log("rotary decode ...")
        result["rotary_decode"] = rotary_decode(torch, sw, args.prompt, 256, use_graph)
    if "small_slack" in only:
        log("small-slack decode ...")
        result["small_slack"] = small_slack(torch, sw, use_graph=use_graph)
    if "chunked" in only:
        for C in (int(x) for x in args.chunk_capacities.split(",")):
            log(f"chunked prefill and verify, C={C} ...")
            result[f"chunked_prefill_c{C}"] = chunked_prefill(torch, sw, C, use_graph=use_graph)
            result[f"verify_c{C}"] = verify_steps(torch, sw, C, use_graph=use_graph)
            result[f"verify_rejection_c{C}"] = verify_with_rejection(torch, sw, C,
                                                                     use_graph=use_graph)
    if "capacity" in only:
        log("capacity sweep ...")
        slacks = tuple(int(x) for x in args.capacity_slacks.split(","))
        pts, comp = capacity_sweep(torch, sw, slacks, use_graph=use_graph)
        result["capacity_sweep"] = {
            "workload": "pages' shape (B=1, 64 Q / 8 KV heads x 64, fp32, W=128), cache at "
                        "T=2048, 800 decode steps, C = W + slack",
            "points": pts}
        if comp:
            result["capacity_sweep"]["compaction_at_C_eq_W"] = comp

    if "copy" in only:
        result["copy_reference"] = copy_reference(torch, args.copy_mib)

    if "cpu" in only and "headline" in only:
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(headline, args.prompt, 400_000, args.cpu_seconds)
        # and at the pages' 8 intra-op threads, for comparison with their figure
        result["cpu_baseline_8_threads"] = cpu_baseline(headline, args.prompt, 400_000,
                                                        args.cpu_seconds / 2, threads=8)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
