"""The SwiGLU clamp and the shared expert on the GPU, against the fp64 oracle.

Readings (see the oracle): R14, with a limit L > 0 every expert's FC1 output is
silu(min(g, L)) * clamp(u, -L, L); R13, the shared expert S adds S(x_t) to y for every
token with weight 1.  The pages fix neither the clamp's form nor its constant (parity
unpinned beyond the oracle's reading); L is chosen here so that it clamps a large share
of the gate and up values, and each test also checks that the clamped result differs
from the unclamped one by far more than the tolerance.

Every FC family is driven: one token (the streaming FC1 and the one-token FC2 with its
combine, whose y the shared expert adds to), token groups on the matrix cores (K = 1024,
2048, 7168), the generic kernels (odd shapes), the prefill GEMMs and the single-call
forward.  The parity rules are those of the other step tests (gpu_util.compare).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from bit_vector_quantised_amd import _lib
from bit_vector_quantised_amd.layer import DeviceLayer, SharedExpert, Step

from gpu_util import Y_TOL, compare, rel_err_rows, run, run_prefill, say, x_tensor
from test_gpu_parity import tiny_variant

pytestmark = pytest.mark.gpu

CONFIGS = {
    # name: config (T tokens, H, I, E, k) and a clamping limit for its magnitudes
    "mini": (synth.Config("mini", 6, 2048, 1024, 16, 4, "bf16", "normal", seed=4242), 0.35),
    "wide": (synth.Config("wide", 40, 7168, 2048, 4, 2, "bf16", "normal", seed=4343), 0.5),
    "odd": (synth.Config("odd", 5, 384, 640, 8, 2, "bf16", "normal", seed=4343), 0.15),
}


def layer(name, limit, mixed=False):
    cfg, _ = CONFIGS[name]
    syn = synth.SynthLayer(cfg, cache=False)
    fm = [synth.FMT_MXFP4 if (mixed and e % 3 == 0) else synth.FMT_VQ2 for e in range(cfg.n_experts)]
    v, _ = tiny_variant(syn, formats=fm)
    dev = DeviceLayer(cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, syn.codebook, syn.router_w, v.expert, fm,
                      swiglu_limit=limit)
    return cfg, syn, v, dev


def clamp_matters(v, x_np, g, top_k, limit, tokens):
    """The clamped oracle is far from the unclamped one on these tokens."""
    x64 = oracle.x_value(x_np, "bf16")[tokens]
    a = oracle.forward(v, x64, top_k, forced_selection=g["ids"][tokens])["y"]
    b = oracle.forward(v, x64, top_k, forced_selection=g["ids"][tokens], swiglu_limit=limit)["y"]
    assert rel_err_rows(a, b).max() > 20 * Y_TOL, "the limit does not clamp enough to be tested"


@pytest.mark.parametrize("name", ["mini", "wide", "odd"])
@pytest.mark.parametrize("mixed", [False, True])
def test_clamped_step(name, mixed):
    cfg, lim = CONFIGS[name]
    _, syn, v, dev = layer(name, lim, mixed)
    x = syn.x()
    toks = list(range(cfg.n_tokens)) if cfg.n_tokens <= 8 else [0, 7, 19, 39]
    say(f"clamp {name} mixed={mixed} L={lim} T={cfg.n_tokens}")
    g = run(dev, x, "bf16")
    assert g["status"] == _lib.OK
    clamp_matters(v, x, g, cfg.top_k, lim, toks)
    r = compare(v, x, "bf16", g, cfg.top_k, tokens=toks, swiglu_limit=lim)
    say(f"  y err {r['y_err']:.2e} h err {r['h_err']:.2e}")
    # one token: the streaming FC1 and the one-token FC2
    g1 = run(dev, x[:1], "bf16")
    assert g1["status"] == _lib.OK
    r1 = compare(v, x[:1], "bf16", g1, cfg.top_k, swiglu_limit=lim)
    say(f"  T=1 y err {r1['y_err']:.2e} h err {r1['h_err']:.2e}")


def test_clamped_prefill_and_forward():
    cfg, lim = CONFIGS["wide"]
    _, syn, v, dev = layer("wide", lim, mixed=True)
    x = syn.x()
    toks = [0, 11, 23, 39]
    say(f"clamp prefill wide T={cfg.n_tokens}")
    g = run_prefill(dev, x, "bf16")
    assert g["status"] == _lib.OK
    x64 = oracle.x_value(x, "bf16")[toks]
    r = oracle.forward(v, x64, cfg.top_k, forced_selection=g["ids"][toks], swiglu_limit=lim)
    e = rel_err_rows(g["y"][toks], r["y"]).max()
    say(f"  prefill y err {e:.2e}")
    assert e <= Y_TOL
    # the single-call forward gives the three-call step's y bit for bit
    st = Step(dev, cfg.n_tokens)
    xt = x_tensor(x, "bf16")
    y3 = st.forward(xt).clone()
    y1 = st.step(xt).clone()
    torch.cuda.synchronize()
    assert st.check()[0] == _lib.OK
    assert torch.equal(y1, y3)


@pytest.mark.parametrize("name", ["mini", "wide", "odd"])
@pytest.mark.parametrize("shared_fmt", [synth.FMT_VQ2, synth.FMT_MXFP4])
def test_shared_expert_added(name, shared_fmt):
    """Routed step, then moe_vq_shared_expert adding S(x) to y: against the oracle with
    O9, at T tokens (matrix-core or generic FC2 with the combine) and at one token (the
    one-token FC2), with the clamp on both the routed and the shared expert."""
    cfg, lim = CONFIGS[name]
    _, syn, v, dev = layer(name, lim, mixed=(shared_fmt == synth.FMT_MXFP4))
    shared = synth.draw_expert(cfg, 1000, shared_fmt)
    se = SharedExpert(cfg.hidden, cfg.inter, syn.codebook, shared, shared_fmt, cfg.n_tokens, swiglu_limit=lim)
    x = syn.x()
    toks = list(range(cfg.n_tokens)) if cfg.n_tokens <= 8 else [0, 7, 19, 39]
    for T in (cfg.n_tokens, 1):
        say(f"shared {name} fmt={shared_fmt} T={T}")
        st = Step(dev, T)
        xt = x_tensor(x[:T], "bf16")
        st.forward(xt)
        y_routed = st.y[:T].clone()
        se.add(xt, st.y[:T])
        torch.cuda.synchronize()
        assert st.check()[0] == _lib.OK and se.check()[0] == _lib.OK
        g = {"ids": st.ids[:T].cpu().numpy().astype(np.int64), "w": st.w[:T].cpu().numpy().astype(np.float64),
             "h": st.h[:T * dev.top_k].cpu().numpy().astype(np.float64).reshape(T, dev.top_k, -1),
             "y": st.y[:T].cpu().numpy().astype(np.float64)}
        tk = [t for t in toks if t < T]
        r = compare(v, x[:T], "bf16", g, cfg.top_k, tokens=tk, swiglu_limit=lim, shared=shared)
        # the shared part alone: y - y_routed against the oracle's S(x)
        ys = (st.y[:T] - y_routed).cpu().numpy().astype(np.float64)[tk]
        es = rel_err_rows(ys, r["ref"]["o_shared"]).max()
        say(f"  y err {r['y_err']:.2e}, shared part err {es:.2e}")
        assert es <= Y_TOL


def test_shared_expert_bf16_and_fp32_x_agree_on_exact_inputs():
    """fp32 x holding bf16 values gives the shared expert's output bit for bit as the bf16
    x (both are staged exactly)."""
    cfg, lim = CONFIGS["mini"]
    syn = synth.SynthLayer(cfg, cache=False)
    shared = synth.draw_expert(cfg, 1001, synth.FMT_VQ2)
    se = SharedExpert(cfg.hidden, cfg.inter, syn.codebook, shared, synth.FMT_VQ2, cfg.n_tokens, swiglu_limit=lim)
    x = syn.x()
    xb = x_tensor(x, "bf16")
    xf = xb.float().contiguous()
    ya = torch.zeros((cfg.n_tokens, cfg.hidden), dtype=torch.float32, device="cuda")
    yb = torch.zeros_like(ya)
    se.add(xb, ya)
    se.add(xf, yb)
    torch.cuda.synchronize()
    assert se.check()[0] == _lib.OK
    assert torch.equal(ya, yb)
