"""Step-sequence drivers shared by the oracle pins and the GPU parity tests.

A scenario owns the synthetic generator, the per-item total lengths and a
per-position ``version`` table (a rejected draft position that is appended
again gets a new version, hence new contents).  Backends hold their own
cache buffers; the oracle backend's state never comes from the GPU.
"""
from __future__ import annotations

import dataclasses

import numpy as np

import oracle
import synth

NAN16 = {synth.F16: 0x7E00, synth.BF16: 0x7FC0}
POISON8 = 127      # poison code of an int8 cache
POISON_FP8 = 0x7E  # poison code of an fp8 E4M3 cache (448)


@dataclasses.dataclass
class Cfg:
    B: int
    Hq: int
    Hkv: int
    D: int
    C: int
    W: int
    dtype: int = synth.F32
    scale: float = 0.0
    softcap: float = 0.0
    seed: int = 1
    v_pos: bool = False
    zero_q: bool = False
    smooth: bool = False       # smooth_softmax: a sink logit of 0
    sink_std: float = 0.0      # > 0: head_sink ~ N(0, sink_std^2) per query head
    rotary: int = -1           # -1 off; 0 pairs (k, k + D/2); 1 interleaved pairs
    rot_rows: int = 4096       # rows of the cos / sin tables
    kv_int8: bool = False      # int8 cache codes with per-tensor scales
    kv_fp8: bool = False       # fp8 E4M3 cache codes with per-tensor scales
    k_scale: float = 0.05
    v_scale: float = 0.04

    def synth(self) -> synth.Synth:
        return synth.Synth(self.seed, self.Hq, self.Hkv, self.D, self.dtype,
                           v_pos_in_elem0=self.v_pos, zero_query=self.zero_q)

    def params(self, S: int, total: int, B: int | None = None):
        return oracle.make_params(self.B if B is None else B, S, self.Hq,
                                  self.Hkv, self.D, self.C, self.W, total,
                                  self.dtype, self.scale, self.softcap,
                                  smooth_softmax=int(self.smooth),
                                  **self.rotary_params(), **self.cache_params())

    @property
    def quantized(self) -> bool:
        return self.kv_int8 or self.kv_fp8

    def cache_params(self):
        if not self.quantized:
            return {}
        return dict(kv_cache_type=2 if self.kv_fp8 else 1, k_scale=self.k_scale,
                    v_scale=self.v_scale)

    @property
    def poison_code(self) -> int:
        return POISON_FP8 if self.kv_fp8 else POISON8

    def cache_array(self, shape):
        """A cache whose every row is poison: NaN, or with 8-bit codes an
        extreme code (int8 127, fp8 448): a read of it moves scores and
        outputs.  Codes are held as int8 bytes."""
        if self.quantized:
            return np.full(shape, self.poison_code, dtype=np.int8)
        return nan_array(shape, self.dtype)

    def rotary_params(self):
        if self.rotary < 0:
            return {}
        return dict(do_rotary=1, rotary_interleaved=self.rotary,
                    rotary_cache_rows=self.rot_rows)

    def rotary_tables(self):
        """(cos, sin) in storage form, or (None, None) without rotary."""
        if self.rotary < 0:
            return None, None
        return synth.rotary_tables(self.rot_rows, self.D, self.dtype)

    def head_sink(self):
        """head_sink in storage form (Hq elements), or None."""
        if self.sink_std <= 0.0:
            return None
        rng = np.random.default_rng(self.seed + 7919)
        return synth.to_storage(rng.normal(0.0, self.sink_std, self.Hq).astype(np.float32),
                                self.dtype)


def nan_array(shape, dtype):
    if dtype == synth.F32:
        return np.full(shape, np.nan, dtype=np.float32)
    return np.full(shape, NAN16[dtype], dtype=np.uint16)


def as_f64(a, dtype):
    return synth.from_storage(np.asarray(a), dtype)


class Versions:
    """version[b][pos]: how many times position pos of item b was re-drawn,
    for positions base .. base + n - 1."""

    def __init__(self, B: int, n: int = 1 << 16, base: int = 0):
        self.v = np.zeros((B, n), dtype=np.int64)
        self.base = base

    def of(self, b: int, pos):
        return self.v[b, np.asarray(pos) - self.base]

    def bump(self, b: int, pos):
        self.v[b, np.asarray(pos) - self.base] += 1


def layout_rows(cfg: Cfg, syn: synth.Synth, b: int, T: int, vers: Versions,
                item_key: int | None = None):
    """Rows the contract puts in [0, L(T)) of item b: (Hkv, L, D) K and V."""
    L = oracle.resident_length(T, cfg.C, cfg.W)
    pos = np.arange(T - L, T)
    ver = vers.of(b, pos)[None, :]
    heads = np.arange(cfg.Hkv)[:, None]
    key = b if item_key is None else item_key
    k = syn.kv_rows(synth.K, key, heads, pos[None, :], ver)
    v = syn.kv_rows(synth.V, key, heads, pos[None, :], ver)
    return L, k, v


def seeded_cache(cfg: Cfg, syn: synth.Synth, Ts, vers: Versions):
    """(B, Hkv, C, D) caches holding the contract layout for lengths Ts and
    NaN in every unspecified row.  With an int8 cache the resident rows are
    seeded codes (uniform in [-100, 100]) and the rest poison codes."""
    shape = (len(Ts), cfg.Hkv, cfg.C, cfg.D)
    if cfg.quantized:
        rng = np.random.default_rng(cfg.seed + 8101)
        K = cfg.cache_array(shape)
        V = cfg.cache_array(shape)

        def codes(n):
            if cfg.kv_int8:
                return rng.integers(-100, 101, size=n)
            # fp8: sign, exponent 0..9, mantissa: finite values up to 7.5
            c = (rng.integers(0, 2, size=n) << 7) | (rng.integers(0, 10, size=n) << 3) | rng.integers(0, 8, size=n)
            return c.astype(np.uint8).view(np.int8)
        for b, T in enumerate(Ts):
            L = oracle.resident_length(int(T), cfg.C, cfg.W)
            K[b, :, :L] = codes((cfg.Hkv, L, cfg.D))
            V[b, :, :L] = codes((cfg.Hkv, L, cfg.D))
        return K, V
    K = nan_array(shape, cfg.dtype)
    V = nan_array(shape, cfg.dtype)
    for b, T in enumerate(Ts):
        L, k, v = layout_rows(cfg, syn, b, int(T), vers)
        K[b, :, :L] = k
        V[b, :, :L] = v
    return K, V


def step_inputs(cfg: Cfg, syn: synth.Synth, P, S: int, vers: Versions):
    P = np.asarray(P, dtype=np.int64)
    ver = np.stack([vers.of(b, P[b] + np.arange(S)) for b in range(len(P))])
    return syn.step_inputs(P, S, ver)


class OracleBackend:
    """Cache state advanced by the oracle alone (in place: present == past)."""

    def __init__(self, cfg: Cfg, K=None, V=None, B: int | None = None):
        B = cfg.B if B is None else B
        shape = (B, cfg.Hkv, cfg.C, cfg.D)
        self.cfg = cfg
        self.K = cfg.cache_array(shape) if K is None else K.copy()
        self.V = cfg.cache_array(shape) if V is None else V.copy()

    def step(self, S, seqlens, q, k, v, bias=None, total=None, bias_bcast=(1, 1),
             position_ids=None):
        seqlens = np.asarray(seqlens, dtype=np.int32)
        total = int(seqlens.max()) + 1 if total is None else total
        p = self.cfg.params(S, total, B=len(seqlens))
        p.bias_dim0_is_batch, p.bias_dim1_is_heads = bias_bcast
        cos, sin = self.cfg.rotary_tables()
        st, out, plan = oracle.forward(p, q, k, v, self.K, self.V, seqlens, bias,
                                       head_sink=self.cfg.head_sink(), cos_cache=cos,
                                       sin_cache=sin, position_ids=position_ids)
        return st, out, plan

    def snapshot(self):
        return self.K.copy(), self.V.copy()

    def restore(self, snap):
        self.K[...] = snap[0]
        self.V[...] = snap[1]
