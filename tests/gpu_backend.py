"""GPU side of the parity tests: device buffers (torch) + calls through the
C ABI of libswgqa via the thin binding.

Storage is raw: float32 for fp32, int16 bit patterns for fp16/bf16, so the
bytes the oracle and the GPU see are identical.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import sliding_window_gqa_02_amd as sw
import synth
from tests.scenario import NAN16, Cfg

DEV = "cuda:0"
GUARD = 4096  # elements of canary before and after every cache buffer


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def to_host(t: torch.Tensor, dtype: int) -> np.ndarray:
    a = t.detach().cpu().numpy()
    return a.view(np.uint16) if dtype != synth.F32 else a


def nan_value(dtype):
    return float("nan") if dtype == synth.F32 else int(np.uint16(NAN16[dtype]).view(np.int16))


def torch_storage(dtype):
    return torch.float32 if dtype == synth.F32 else torch.int16


INT8 = "int8"  # cache storage tag of an int8 cache


def cache_poison(cfg: Cfg):
    return cfg.poison_code if cfg.quantized else nan_value(cfg.dtype)


class GuardedCache:
    """A (B, Hkv, C, D) cache inside a larger allocation whose margins hold a
    canary pattern; `intact()` checks nothing was written outside."""

    CANARY32 = 0x5A5AA5A5

    def __init__(self, shape, dtype, poison=None):
        n = int(np.prod(shape))
        if dtype == INT8:
            self.flat = torch.empty(n + 2 * GUARD, dtype=torch.int8, device=DEV)
            self.flat.fill_(0x5A)
        else:
            self.flat = torch.empty(n + 2 * GUARD, dtype=torch_storage(dtype), device=DEV)
            if dtype == synth.F32:
                self.flat.view(torch.int32).fill_(self.CANARY32)
            else:
                self.flat.fill_(0x2BCD)
        self.t = self.flat[GUARD:GUARD + n].view(*shape)
        self.t.fill_(poison if poison is not None else nan_value(dtype))
        self.dtype = dtype

    def intact(self) -> bool:
        g = torch.cat([self.flat[:GUARD], self.flat[-GUARD:]])
        if self.dtype == INT8:
            return bool((g == 0x5A).all())
        if self.dtype == synth.F32:
            return bool((g.view(torch.int32) == self.CANARY32).all())
        return bool((g == 0x2BCD).all())


class GpuBackend:
    """Cache state advanced by libswgqa.  mode 'shared': present == past (in
    place); mode 'separate': ping-pong between two buffers."""

    def __init__(self, cfg: Cfg, K=None, V=None, B=None, mode="shared"):
        B = cfg.B if B is None else B
        self.cfg = cfg
        self.B = B
        self.mode = mode
        shape = (B, cfg.Hkv, cfg.C, cfg.D)
        ct = INT8 if cfg.quantized else cfg.dtype
        self.bufs = [(GuardedCache(shape, ct, cache_poison(cfg)), GuardedCache(shape, ct, cache_poison(cfg)))]
        if mode == "separate":
            self.bufs.append((GuardedCache(shape, ct, cache_poison(cfg)),
                              GuardedCache(shape, ct, cache_poison(cfg))))
        if K is not None:
            self.bufs[0][0].t.copy_(to_dev(K))
            self.bufs[0][1].t.copy_(to_dev(V))
        self.cur = 0
        self.ws = None
        self.ws_bytes = 0
        self.T = None  # per-item lengths, tracked by the caller via step()

    @property
    def K(self):
        return self.bufs[self.cur][0].t

    @property
    def V(self):
        return self.bufs[self.cur][1].t

    def intact(self) -> bool:
        return all(c.intact() for pair in self.bufs for c in pair)

    def _workspace(self, p):
        need = sw.workspace_size(p)
        assert need > 0
        if self.ws is None or need > self.ws_bytes:
            self.ws = torch.zeros(need // 4 + 64, dtype=torch.int32, device=DEV)
            self.ws_bytes = need
            sw.workspace_init(self.ws)
        return self.ws

    def poison_unspecified(self, P):
        """Rows [L(P_b), C) of the current cache are unspecified: NaN them so
        that a kernel reading one shows up in the outputs."""
        nv = cache_poison(self.cfg)
        for b, Pb in enumerate(np.asarray(P)):
            if Pb < 0:
                continue
            L = oracle.resident_length(int(Pb), self.cfg.C, self.cfg.W)
            self.K[b, :, L:].fill_(nv)
            self.V[b, :, L:].fill_(nv)

    def step(self, S, seqlens, q, k, v, bias=None, total=None, bias_bcast=(1, 1),
             poison=True, position_ids=None):
        cfg = self.cfg
        seqlens = np.asarray(seqlens, dtype=np.int32)
        B = len(seqlens)
        total = int(seqlens.max()) + 1 if total is None else total
        p = sw.make_params(B, S, cfg.Hq, cfg.Hkv, cfg.D, cfg.C, cfg.W, total,
                           cfg.dtype, cfg.scale, cfg.softcap, *bias_bcast,
                           smooth_softmax=int(cfg.smooth), **cfg.rotary_params(),
                           **cfg.cache_params())
        if poison:
            self.poison_unspecified(seqlens.astype(np.int64) + 1 - S)
        dq, dk, dv = to_dev(q), to_dev(k), to_dev(v)
        dbias = None if bias is None else to_dev(bias)
        dseq = to_dev(seqlens)
        out = torch.full(dq.shape, nan_value(cfg.dtype), dtype=torch_storage(cfg.dtype), device=DEV)
        ws = self._workspace(p)
        pk, pv = self.K, self.V
        if self.mode == "separate":
            nxt = 1 - self.cur
            prk, prv = self.bufs[nxt][0].t, self.bufs[nxt][1].t
            prk.fill_(cache_poison(cfg))
            prv.fill_(cache_poison(cfg))
        else:
            nxt = self.cur
            prk, prv = pk, pv
        sink = cfg.head_sink()
        dsink = None if sink is None else to_dev(sink)
        cos, sin = cfg.rotary_tables()
        dcos = None if cos is None else to_dev(cos)
        dsin = None if sin is None else to_dev(sin)
        dpos = None if position_ids is None else to_dev(np.asarray(position_ids, np.int64))
        sw.forward(p, dq, dk, dv, pk, pv, dseq, dbias, out, prk, prv, ws, head_sink=dsink,
                   cos_cache=dcos, sin_cache=dsin, position_ids=dpos)
        torch.cuda.synchronize()
        self.cur = nxt
        status = sw.device_status(ws, clear=True)
        return status, to_host(out, cfg.dtype)

    def counters_zero(self) -> bool:
        """The per-slice arrival counters (workspace bytes [256, 16384)) are
        zero between calls."""
        return self.ws is None or int(self.ws[64:4096].abs().sum().item()) == 0

    def present_host(self):
        if self.cfg.quantized:
            return self.K.cpu().numpy(), self.V.cpu().numpy()
        return to_host(self.K, self.cfg.dtype), to_host(self.V, self.cfg.dtype)

    def snapshot(self):
        return self.K.clone(), self.V.clone()

    def restore(self, snap):
        self.K.copy_(snap[0])
        self.V.copy_(snap[1])
