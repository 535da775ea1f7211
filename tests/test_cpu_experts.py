"""The CPU miss path (moe_vq_cpu_experts): routed experts computed on the host cores from a
host slot pool, against the fp64 oracle.  No GPU is needed: the call is host code of the
C-ABI library.  Decoding is exact and the products and sums are fp32, so each token's
output matches the oracle to fp32 rounding (checked at 2e-5 of max |y|); the thread count
does not change a bit."""
import ctypes

import numpy as np
import pytest

import oracle
import synth

mvq = pytest.importorskip("bit_vector_quantised_amd")
from bit_vector_quantised_amd import _lib  # noqa: E402
from bit_vector_quantised_amd.layer import pack_slot  # noqa: E402

Y_TOL = 2e-5


class HostLayer:
    """Every expert of a synthetic layer packed into one host pool (the device pool's slot
    layout)."""

    def __init__(self, cfg, formats=None, mutate=None):
        self.syn = synth.SynthLayer(cfg)
        self.cfg = cfg
        self.codebook, self.router_w = self.syn.codebook, self.syn.router_w
        fm = list(self.syn.formats) if formats is None else list(formats)
        self.formats = fm
        self.experts = {e: self.syn.expert_as(e, fm[e]) for e in range(cfg.n_experts) if fm[e] != synth.FMT_ABSENT}
        if mutate:
            mutate(self.experts)
        bufs, offs, off = [], [], 0
        for e in range(cfg.n_experts):
            if fm[e] == synth.FMT_ABSENT:
                offs.append(0)
                continue
            b = pack_slot(self.experts[e], cfg.hidden, cfg.inter, fm[e])
            offs.append(off)
            bufs.append(b)
            off += b.size
        self.pool = np.concatenate(bufs) if bufs else np.zeros(256, np.uint8)
        self.slots = (_lib.Slot * cfg.n_experts)(*[_lib.Slot(offs[e], int(fm[e]), 0) for e in range(cfg.n_experts)])
        self.c = _lib.Layer(cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, 0, 0, 0, 0, 0)

    def expert(self, e):
        return self.experts[e]

    def run(self, x, x_dtype, ids, w, compute, threads=4, y=None):
        T = x.shape[0]
        x = np.ascontiguousarray(x)
        ids32 = np.ascontiguousarray(ids, dtype=np.int32)
        w32 = np.ascontiguousarray(w, dtype=np.float32)
        comp = np.zeros(self.cfg.n_experts, np.uint8)
        comp[list(compute)] = 1
        y = np.zeros((T, self.cfg.hidden), np.float32) if y is None else y
        cb = np.ascontiguousarray(self.codebook).view(np.uint16)
        rc = _lib.raw().moe_vq_cpu_experts(
            ctypes.byref(self.c), self.pool.ctypes.data, self.pool.size, self.slots, cb.ctypes.data, x.ctypes.data,
            _lib.BF16 if x_dtype == "bf16" else _lib.F32, T, ids32.ctypes.data, w32.ctypes.data, comp.ctypes.data,
            y.ctypes.data, threads)
        return rc, y


def _oracle_part(layer, x64, ids, compute, swiglu_limit=0.0):
    """y restricted to the pairs whose expert is in `compute`, from the oracle (with the
    given selection and its renormalised weights)."""
    r = oracle.forward(layer, x64, ids.shape[1], forced_selection=ids, swiglu_limit=swiglu_limit)
    keep = np.isin(ids, list(compute))[:, :, None]
    return (r["w"][:, :, None] * r["o"] * keep).sum(axis=1), r["w"]


def _check(y, ref):
    den = np.abs(ref).max(axis=1)
    err = np.abs(y.astype(np.float64) - ref).max(axis=1) / np.where(den > 0, den, 1)
    assert err.max() <= Y_TOL, err.max()
    return err.max()


def test_all_experts_tiny_fp32():
    L = HostLayer(synth.PRESETS["tiny"])
    x = L.syn.x()
    x64 = oracle.x_value(x, "f32")
    ids = oracle.topk(oracle.router_logits(L.router_w, x64), 2)
    ref, w = _oracle_part(L, x64, ids, range(8))
    rc, y = L.run(x, "f32", ids, w, range(8))
    assert rc == _lib.OK
    _check(y, ref)


def test_subset_mixed_formats_and_accumulation():
    fm = [synth.FMT_MXFP4 if e % 2 else synth.FMT_VQ2 for e in range(8)]
    L = HostLayer(synth.PRESETS["tiny"], formats=fm)
    x = L.syn.x(n=7, stream=3)
    x64 = oracle.x_value(x, "f32")
    ids = oracle.topk(oracle.router_logits(L.router_w, x64), 2)
    used = sorted(set(ids.ravel().tolist()))
    part = used[::2]
    ref, w = _oracle_part(L, x64, ids, part)
    base = np.full((7, 256), 0.25, np.float32)  # y is accumulated into
    rc, y = L.run(x, "f32", ids, w, part, y=base.copy())
    assert rc == _lib.OK
    _check(y - base, ref)


def test_mini_bf16_threads_do_not_change_bits():
    cfg = synth.Config("mini", 5, 2048, 1024, 16, 4, "bf16", "normal", seed=4242)
    L = HostLayer(cfg)
    x = L.syn.x(n=5, stream=9)
    x64 = oracle.x_value(x, "bf16")
    ids = oracle.topk(oracle.router_logits(L.router_w, x64), 4)
    used = sorted(set(ids.ravel().tolist()))
    ref, w = _oracle_part(L, x64, ids, used)
    rc1, y1 = L.run(x, "bf16", ids, w, used, threads=1)
    rc8, y8 = L.run(x, "bf16", ids, w, used, threads=8)
    assert rc1 == rc8 == _lib.OK
    assert np.array_equal(y1, y8)
    _check(y1, ref)


def test_extreme_mxfp4_exponents():
    def shift(experts):
        for e, ex in experts.items():
            if int(ex["format"]) == synth.FMT_MXFP4:
                ex["e8m0_g"] = (ex["e8m0_g"].astype(np.int64) + 25).astype(np.uint8)
                ex["e8m0_d"] = (ex["e8m0_d"].astype(np.int64) - 17).astype(np.uint8)
    L = HostLayer(synth.PRESETS["tiny"], formats=[synth.FMT_MXFP4] * 8, mutate=shift)
    x = L.syn.x(n=3, stream=4)
    x64 = oracle.x_value(x, "f32")
    ids = oracle.topk(oracle.router_logits(L.router_w, x64), 2)
    ref, w = _oracle_part(L, x64, ids, range(8))
    rc, y = L.run(x, "f32", ids, w, range(8))
    assert rc == _lib.OK
    _check(y, ref)


def test_errors():
    fm = list(synth.SynthLayer(synth.PRESETS["tiny"]).formats)
    fm[3] = synth.FMT_ABSENT
    L = HostLayer(synth.PRESETS["tiny"], formats=fm)
    x = L.syn.x(n=2)
    ids = np.array([[3, 1], [0, 2]], np.int32)
    w = np.full((2, 2), 0.5, np.float32)
    y0 = np.full((2, 256), 7.0, np.float32)
    rc, y = L.run(x, "f32", ids, w, [3], y=y0.copy())
    assert rc == _lib.ENOTRESIDENT and np.all(y == 7.0)  # nothing added
    rc, y = L.run(x, "f32", ids, w, [1, 2], y=y0.copy())   # the absent expert is not asked for
    assert rc == _lib.OK
    rc, _ = L.run(x, "f32", np.array([[9, 1], [0, 2]], np.int32), w, [1])
    assert rc == _lib.EINVAL
    rc, _ = L.run(x, "f32", ids, w, [1], threads=0)
    assert rc == _lib.EINVAL
    rc, _ = L.run(x[:0], "f32", ids[:0], w[:0], [1])
    assert rc == _lib.OK


def test_swiglu_clamp_on_the_host():
    """The layer's SwiGLU clamp (reading R14) applies on the host path too: against the
    oracle with the same limit, chosen so that it clamps, and different from no clamp."""
    L = HostLayer(synth.PRESETS["tiny"])
    x = L.syn.x(n=5, stream=4)
    x64 = oracle.x_value(x, "f32")
    ids = oracle.topk(oracle.router_logits(L.router_w, x64), 2)
    ref0, w = _oracle_part(L, x64, ids, range(8))
    lim = 0.02
    ref, _ = _oracle_part(L, x64, ids, range(8), swiglu_limit=lim)
    assert np.abs(ref - ref0).max() > 0.05 * np.abs(ref0).max()
    L.c.swiglu_limit = lim
    rc, y = L.run(x, "f32", ids, w, range(8))
    assert rc == _lib.OK
    _check(y, ref)
    L.c.swiglu_limit = -1.0
    rc, _ = L.run(x, "f32", ids, w, range(8))
    assert rc == _lib.EINVAL
