"""swgqa_forward_noalloc (the library's static scratch as workspace) against
swgqa_forward (a caller's workspace), both through the C ABI: calls in a row
on the same GPU, each later one smaller than the first, every output and
every present byte equal.  The first call is a multi-token step with key
splits (partials in the scratch), then a decode step whose query tiles
compact in place through the slice counters, then a long-window decode
merged from key splits; device item errors reach the caller's status word.
"""
from __future__ import annotations

import numpy as np
import pytest

import synth
from tests.parity import say
from tests.scenario import Cfg, Versions, seeded_cache, step_inputs

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sliding_window_gqa_02_amd as sw
    sw.load()


def _bias(cfg, syn, P, S, total):
    bias = syn.bias_f32(np.arange(len(P)), P, S, total)
    return synth.to_storage(bias, cfg.dtype)


def _run_both(cfg, P, S, with_bias=False, seqlens=None):
    """The same step through both entry points on equal copies of a seeded
    cache; returns (outputs, presents) of each and the status words."""
    import sliding_window_gqa_02_amd as sw
    from tests.gpu_backend import to_dev
    syn = cfg.synth()
    vers = Versions(len(P), n=int(max(P)) + S + 1)
    K, V = seeded_cache(cfg, syn, P, vers)
    q, k, v = step_inputs(cfg, syn, P, S, vers)
    seq = (np.asarray(P) + S - 1).astype(np.int32) if seqlens is None else seqlens
    total = int(max(P)) + S
    bias = _bias(cfg, syn, P, S, total) if with_bias else None
    p = sw.make_params(len(P), S, cfg.Hq, cfg.Hkv, cfg.D, cfg.C, cfg.W, total, cfg.dtype,
                       cfg.scale, cfg.softcap)
    dq, dk, dv, dseq = to_dev(q), to_dev(k), to_dev(v), to_dev(seq)
    dbias = None if bias is None else to_dev(bias)
    res = {}
    for which in ("forward", "noalloc"):
        Kd, Vd = to_dev(K), to_dev(V)
        out = torch.zeros_like(dq)
        if which == "forward":
            ws = torch.zeros(sw.workspace_size(p) // 4 + 64, dtype=torch.int32, device="cuda:0")
            sw.workspace_init(ws)
            st = sw.forward_status(p, dq, dk, dv, Kd, Vd, dseq, dbias, out, Kd, Vd, ws)
            assert st == sw.OK
            torch.cuda.synchronize()
            word = sw.device_status(ws)
        else:
            status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
            st = sw.forward_noalloc_status(p, dq, dk, dv, Kd, Vd, dseq, dbias, out, Kd, Vd,
                                           device_status=status)
            assert st == sw.OK, sw.status_string(st)
            torch.cuda.synchronize()
            word = sw.ERR_DEVICE_INPUT if int(status.item()) != 0 else sw.OK
        res[which] = (out.cpu().numpy(), Kd.cpu().numpy(), Vd.cpu().numpy(), word)
    return res


def _assert_equal(res, what):
    fo, fk, fv, fw = res["forward"]
    no, nk, nv, nw = res["noalloc"]
    assert fw == nw, f"{what}: status {fw} vs {nw}"
    assert np.array_equal(fo.view(np.uint8), no.view(np.uint8)), f"{what}: outputs differ"
    assert np.array_equal(fk.view(np.uint8), nk.view(np.uint8)), f"{what}: present_key differs"
    assert np.array_equal(fv.view(np.uint8), nv.view(np.uint8)), f"{what}: present_value differs"


def test_noalloc_equals_forward_on_calls_in_a_row():
    import sliding_window_gqa_02_amd as sw
    # 1: multi-token steps with key splits over a windowed cache, with bias
    big = Cfg(B=4, Hq=32, Hkv=8, D=128, C=1032, W=1024, seed=301, dtype=synth.F16)
    p_big = sw.make_params(4, 32, 32, 8, 128, 1032, 1024, 5000, synth.F16)
    assert 1 << 20 < sw.workspace_size(p_big) <= 32 << 20
    say("noalloc call 1: B=4 S=32 chunk step with key splits")
    _assert_equal(_run_both(big, [1500, 2047, 3333, 4000], 32, with_bias=True), "call 1")
    # 2: smaller -- decode over few slices, query tiles counted for the
    # in-place compaction (T = 21 compacts: L(20) = 20, L(21) = 12 + 0)
    small = Cfg(B=1, Hq=16, Hkv=2, D=64, C=20, W=12, seed=302)
    say("noalloc call 2: decode, counted compaction")
    for P in (19, 20, 21, 27):
        _assert_equal(_run_both(small, [P], 1), f"call 2 P={P}")
    # 3: smaller again -- a long window over one slice: key splits merged by
    # the step tail
    long = Cfg(B=1, Hq=4, Hkv=1, D=128, C=1600, W=1500, seed=303, dtype=synth.BF16,
               softcap=50.0)
    say("noalloc call 3: long-window decode, key splits")
    _assert_equal(_run_both(long, [1700], 1), "call 3")
    # an invalid item (seqlens_k + 1 < S) reaches the caller's status word
    say("noalloc: invalid item flagged")
    bad = _run_both(Cfg(B=2, Hq=4, Hkv=2, D=16, C=12, W=8, seed=304), [5, 5], 3,
                    seqlens=np.array([7, 0], np.int32))
    _assert_equal(bad, "invalid item")
    assert bad["noalloc"][3] == sw.ERR_DEVICE_INPUT


def test_noalloc_refuses_steps_beyond_the_scratch():
    import sliding_window_gqa_02_amd as sw
    t = torch.zeros(4096, dtype=torch.float32, device="cuda:0")
    seq = torch.zeros(8, dtype=torch.int32, device="cuda:0")
    p = sw.make_params(8, 1024, 32, 8, 128, 2048, 1024, 1024, synth.BF16, do_rotary=1,
                       rotary_cache_rows=2048)
    assert sw.workspace_size(p) > 32 << 20
    assert sw.forward_noalloc_status(p, t, t, t, t, t, seq, None, t, t, t, cos_cache=t,
                                     sin_cache=t) == sw.ERR_SCRATCH
    torch.cuda.synchronize()
