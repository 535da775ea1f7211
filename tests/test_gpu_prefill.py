"""GPU parity of the prefill form (tokens grouped per expert, FC1 and FC2 as grouped
matrix-core GEMMs) against the fp64 oracle: same selection rule, weights within 1e-5,
per token max |y - y_oracle| <= 1e-2 max |y_oracle|.  The prefill operands are fp16
(activations with a power-of-two factor per token or pair, weights decoded and
scaled in fp16), inside that tolerance."""
import numpy as np
import pytest
import torch

import oracle
import synth
from bit_vector_quantised_amd import _lib
from bit_vector_quantised_amd.layer import DeviceLayer, Step

from gpu_util import compare, run, run_prefill, say, x_tensor
from test_gpu_parity import MINI, tiny_variant

pytestmark = pytest.mark.gpu

ODD = synth.Config("odd", 5, 384, 640, 8, 2, "bf16", "normal", seed=4343)


@pytest.fixture(scope="module")
def tiny():
    syn = synth.SynthLayer(synth.PRESETS["tiny"])
    return syn, DeviceLayer.from_synth(syn)


@pytest.fixture(scope="module")
def mini():
    syn = synth.SynthLayer(MINI)
    return syn, DeviceLayer.from_synth(syn)


@pytest.fixture(scope="module")
def odd():
    syn = synth.SynthLayer(ODD)
    return syn, DeviceLayer.from_synth(syn)


def test_prefill_tiny(tiny):
    syn, dev = tiny
    x = syn.x()
    say("prefill tiny")
    g = run_prefill(dev, x, "f32")
    assert g["status"] == _lib.OK
    compare(syn, x, "f32", g, syn.cfg.top_k, check_h=False)


@pytest.mark.parametrize("T", [1, 3, 65, 300])
def test_prefill_tiny_token_counts(tiny, T):
    syn, dev = tiny
    x = syn.x(n=T, stream=60 + T)
    say(f"prefill tiny T={T}")
    g = run_prefill(dev, x, "f32")
    assert g["status"] == _lib.OK
    compare(syn, x, "f32", g, syn.cfg.top_k, check_h=False)


@pytest.mark.parametrize("T", [1, 70, 300])
def test_prefill_mini(mini, T):
    syn, dev = mini
    x = syn.x(n=T, stream=70 + T)
    say(f"prefill mini T={T}")
    g = run_prefill(dev, x, "bf16")
    assert g["status"] == _lib.OK
    compare(syn, x, "bf16", g, MINI.top_k, check_h=False)


def test_prefill_agrees_with_decode_path(mini):
    syn, dev = mini
    x = syn.x(n=40, stream=77)
    st = Step(dev, 40)
    gp = run_prefill(dev, x, "bf16", step=st)
    yp = gp["y"].copy()
    gd = run(dev, x, "bf16", step=st)
    assert np.array_equal(gp["ids"], gd["ids"])
    err = np.abs(yp - gd["y"]).max(axis=1) / np.abs(gd["y"]).max(axis=1)
    assert err.max() <= 1e-2


def test_prefill_mixed_formats(mini):
    syn, _ = mini
    fm = [synth.FMT_MXFP4 if e % 3 == 0 else synth.FMT_VQ2 for e in range(MINI.n_experts)]
    v, dev = tiny_variant(syn, formats=fm)
    x = syn.x(n=150, stream=80)
    say("prefill mini mixed")
    g = run_prefill(dev, x, "bf16")
    assert g["status"] == _lib.OK
    compare(v, x, "bf16", g, MINI.top_k, check_h=False)


def test_prefill_partly_filled_token_tiles(mini):
    # A tile holds up to 64 tokens of one expert; the kernels multiply only its 16-token
    # blocks that hold tokens.  Token counts chosen so that tiles with 1, 2, 3 and 4 such
    # blocks occur for VQ2 and MXFP4 experts, every token compared with the oracle.
    syn, _ = mini
    fm = [synth.FMT_MXFP4 if e % 3 == 0 else synth.FMT_VQ2 for e in range(MINI.n_experts)]
    v, dev = tiny_variant(syn, formats=fm)
    seen = set()
    for T in (40, 100, 170, 300):
        x = syn.x(n=T, stream=110 + T)
        say(f"prefill mini mixed T={T}")
        g = run_prefill(dev, x, "bf16")
        assert g["status"] == _lib.OK
        compare(v, x, "bf16", g, MINI.top_k, check_h=False)
        counts = np.bincount(g["ids"].reshape(-1), minlength=MINI.n_experts)
        for e, c in enumerate(counts):
            sizes = [64] * (int(c) // 64) + ([int(c) % 64] if c % 64 else [])
            seen |= {(fm[e], -(-n // 16)) for n in sizes}
    for f in (synth.FMT_VQ2, synth.FMT_MXFP4):
        assert {b for (ff, b) in seen if ff == f} == {1, 2, 3, 4}


def test_prefill_ragged_row_tiles(odd):
    # H=384: the FC2 tile of 256 rows is ragged; K=384 / 640 are not multiples of 1024
    syn, dev = odd
    for T in (5, 90):
        x = syn.x(n=T, stream=90 + T)
        say(f"prefill odd T={T}")
        g = run_prefill(dev, x, "bf16")
        assert g["status"] == _lib.OK
        compare(syn, x, "bf16", g, ODD.top_k, check_h=False)


def test_prefill_absent_expert_is_reported_and_left_out(tiny):
    syn, _ = tiny
    x = syn.x(n=40, stream=99)
    x64 = oracle.x_value(x, "f32")
    ids = oracle.topk(oracle.router_logits(syn.router_w, x64), syn.cfg.top_k)
    gone = int(np.bincount(ids.reshape(-1)).argmax())
    fm = list(syn.formats)
    fm[gone] = synth.FMT_ABSENT
    v, dev = tiny_variant(syn, formats=fm)
    g = run_prefill(dev, x, "f32")
    assert g["status"] == _lib.ENOTRESIDENT and g["info"] == gone
    r = oracle.forward(syn, x64, syn.cfg.top_k, forced_selection=g["ids"])
    keep = (g["ids"] != gone)[:, :, None]
    y_ref = (r["w"][:, :, None] * r["o"] * keep).sum(axis=1)
    err = np.abs(g["y"] - y_ref).max(axis=1) / np.abs(y_ref).max(axis=1)
    assert err.max() <= 1e-2


@pytest.fixture(scope="module")
def p4096():
    cfg = synth.PRESETS["p4096"]
    say("building p4096 pool")
    dev = DeviceLayer.from_synth(synth.SynthLayer(cfg, cache=False))
    yield synth.SynthLayer(cfg), dev
    del dev
    torch.cuda.empty_cache()


def test_p4096_prefill_sampled_tokens(p4096):
    syn, dev = p4096
    x = syn.x()
    say("p4096 prefill")
    g = run_prefill(dev, x, "bf16")
    assert g["status"] == _lib.OK
    info = g["step"].info(4096)
    assert info["n_pairs"] == 4096 * 8
    hot = int(np.bincount(g["ids"].reshape(-1)).argmax())
    tokens = {0, 1, 2047, 4095} | {int(t) for t in np.nonzero((g["ids"] == hot).any(axis=1))[0][:4]}
    rng = np.random.default_rng(4096)
    tokens |= {int(t) for t in rng.choice(4096, size=40, replace=False)}
    tokens = sorted(tokens)[:40]
    assert len(tokens) >= 32
    res = compare(syn, x, "bf16", g, 8, tokens=tokens, check_h=False)
    say("p4096", {k: v for k, v in res.items() if k != "ref"})


def test_max_tokens_decode_and_prefill(p4096):
    # The largest token count a step takes (65536 tokens, 524288 routed pairs) at the full
    # layer shape: per-pair outputs then hold 3.8e9 floats, past 32-bit indexing.  The
    # decode path (route, FC1, FC2) and prefill run on all tokens; sampled tokens, the
    # first and last among them, are compared with the oracle.
    syn, dev = p4096
    T = 65536
    assert T == 65536 and T * 8 * 7168 > 2 ** 31
    say("drawing 65536 tokens")
    x = syn.x(n=T, stream=65536)
    xt = x_tensor(x, "bf16")
    st = Step(dev, T)
    rng = np.random.default_rng(65536)
    tokens = np.array(sorted({0, 1, T // 2, T - 2, T - 1} | {int(t) for t in rng.choice(T, 11, replace=False)}))
    k = dev.top_k
    ti = torch.from_numpy(tokens).cuda()
    pi = (ti[:, None] * k + torch.arange(k, device=ti.device)[None, :]).reshape(-1)

    def sampled(with_h):
        torch.cuda.synchronize()
        g = {"ids": st.ids[ti].cpu().numpy().astype(np.int64), "w": st.w[ti].cpu().numpy().astype(np.float64),
             "y": st.y[ti].cpu().numpy().astype(np.float64)}
        if with_h:
            g["h"] = st.h[pi].cpu().numpy().astype(np.float64).reshape(len(tokens), k, -1)
        return g

    say("T=65536 decode")
    st.forward(xt)
    status, _ = st.check()
    assert status == _lib.OK
    assert st.info(T)["n_pairs"] == T * k
    g = sampled(True)
    compare(syn, x[tokens], "bf16", g, k)
    say("T=65536 prefill")
    st.route(xt)
    st.prefill(xt)
    status, _ = st.check()
    assert status == _lib.OK
    gp = sampled(False)
    assert np.array_equal(gp["ids"], g["ids"])
    compare(syn, x[tokens], "bf16", gp, k, check_h=False)
    del st, xt
    torch.cuda.empty_cache()
