"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Decode is compared bit for bit; routing selects the same experts (or, at a near
tie within the fp32 dot-product error bound, an equally valid set that the oracle
then uses); weights within 1e-5; per token max |y - y_oracle| <= 1e-2 max |y_oracle|.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from bit_vector_quantised_amd import _lib
from bit_vector_quantised_amd.layer import DeviceLayer, Step

from gpu_util import bf16_rne_bits, compare, decode_on_gpu, run, run_prefill, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tiny():
    syn = synth.SynthLayer(synth.PRESETS["tiny"])
    return syn, DeviceLayer.from_synth(syn)


def tiny_variant(syn, formats=None, top_k=None, mutate=None):
    cfg = syn.cfg
    experts = {e: {k: np.array(v, copy=True) for k, v in syn.expert(e).items()} for e in range(cfg.n_experts)}
    fm = syn.formats if formats is None else np.asarray(formats)
    for e in range(cfg.n_experts):
        if int(fm[e]) != synth.FMT_ABSENT and int(fm[e]) != int(experts[e]["format"]):
            experts[e] = synth.draw_expert(cfg, e, int(fm[e]))
    if mutate:
        mutate(experts)

    class V:
        pass
    v = V()
    v.cfg, v.codebook, v.router_w, v.formats = cfg, syn.codebook, syn.router_w, fm
    v.expert = lambda e: experts[e]
    k = cfg.top_k if top_k is None else top_k
    dev = DeviceLayer(cfg.hidden, cfg.inter, cfg.n_experts, k, syn.codebook, syn.router_w, v.expert, fm)
    return v, dev


# ---------------------------------------------------------------------------------
# P1: decode, bit for bit
# ---------------------------------------------------------------------------------

def _check_decode(syn, dev, experts, mats=(0, 1, 2), rows=None):
    for e in experts:
        Wg, Wu, Wd = oracle.decode_expert(syn.expert(e), syn.codebook)
        for mat, W in zip((0, 1, 2), (Wg, Wu, Wd)):
            if mat not in mats:
                continue
            ref32 = W.astype(np.float32)
            assert np.array_equal(ref32.astype(np.float64), W), "decode not exact in fp32"
            got, st = decode_on_gpu(dev, e, mat, _lib.F32)
            assert st == _lib.OK
            sl = slice(None) if rows is None else rows
            assert np.array_equal(got[sl].view(np.uint32), ref32[sl].view(np.uint32)), (e, mat)
            gotb, st = decode_on_gpu(dev, e, mat, _lib.BF16)
            assert np.array_equal(gotb[sl].view(np.uint16), bf16_rne_bits(ref32[sl])), (e, mat, "bf16")


def test_decode_vq2_bitexact_tiny(tiny):
    syn, dev = tiny
    say("decode vq2 tiny")
    _check_decode(syn, dev, range(syn.cfg.n_experts))


def test_decode_mxfp4_bitexact_tiny(tiny):
    syn, _ = tiny
    v, dev = tiny_variant(syn, formats=[synth.FMT_MXFP4] * syn.cfg.n_experts)
    say("decode mxfp4 tiny")
    _check_decode(v, dev, range(syn.cfg.n_experts))


def test_decode_reports_absent_slot(tiny):
    syn, _ = tiny
    fm = list(syn.formats)
    fm[3] = synth.FMT_ABSENT
    v, dev = tiny_variant(syn, formats=fm)
    _, st = decode_on_gpu(dev, 3, 0, _lib.F32)
    assert st == _lib.ENOTRESIDENT
    _, st = decode_on_gpu(dev, 2, 0, _lib.F32)
    assert st == _lib.OK


# ---------------------------------------------------------------------------------
# Whole step on the tiny layer
# ---------------------------------------------------------------------------------

def test_tiny_step_parity_and_determinism(tiny):
    syn, dev = tiny
    x = syn.x()
    say("tiny step T=4 f32")
    g = run(dev, x, "f32")
    assert g["status"] == _lib.OK
    res = compare(syn, x, "f32", g, syn.cfg.top_k)
    say("tiny", {k: v for k, v in res.items() if k != "ref"})
    g2 = run(dev, x, "f32", step=g["step"])
    assert np.array_equal(g["y"], g2["y"]) and np.array_equal(g["ids"], g2["ids"])
    info = g["step"].info(4)
    assert info["experts"] == sorted(set(g["ids"].reshape(-1).tolist()))
    assert info["n_pairs"] == 4 * syn.cfg.top_k


@pytest.mark.parametrize("T", [1, 2, 3, 5, 7, 16])
def test_tiny_ragged_token_counts(tiny, T):
    syn, dev = tiny
    x = syn.x(n=T, stream=10 + T)
    say(f"tiny step T={T}")
    g = run(dev, x, "f32")
    assert g["status"] == _lib.OK
    compare(syn, x, "f32", g, syn.cfg.top_k)


def test_tiny_bf16_activations(tiny):
    syn, dev = tiny
    xb = synth.f64_to_bf16_bits(syn.x(n=6, stream=3).astype(np.float64))
    say("tiny step bf16")
    g = run(dev, xb, "bf16")
    compare(syn, xb, "bf16", g, syn.cfg.top_k)


def test_empty_batch_is_a_no_op(tiny):
    """Zero tokens: every compute call returns OK without launching or writing anything
    (null pointers are allowed then), and the next step is unaffected."""
    syn, dev = tiny
    st = Step(dev, 4)
    bufs = (st.ids, st.w, st.h, st.y)
    for b in bufs:
        b.fill_(7)
    L, s = dev.c, st.stream()
    _lib.route_topk(L, 0, _lib.F32, 0, 0, 0, 0, 0, s)
    _lib.fc1_silu(L, 0, _lib.BF16, 0, 0, 0, 0, s)
    _lib.fc2_combine(L, 0, 0, 0, 0, 0, s)
    _lib.prefill_gemm(L, 0, _lib.F32, 0, 0, 0, 0, s)
    _lib.forward(L, 0, _lib.F32, 0, 0, 0, 0, 0, 0, 0, s)
    _lib.forward_static(L, 0, _lib.BF16, 0, 0, 0, 0, 0, 0, s)
    torch.cuda.synchronize()
    assert all(bool((b == 7).all()) for b in bufs)
    x = syn.x()
    g = run(dev, x, "f32", step=st)
    assert g["status"] == _lib.OK
    compare(syn, x, "f32", g, syn.cfg.top_k)


def test_zero_input_selects_lowest_ids(tiny):
    """x = 0: all logits tie, so the experts are 0..k-1 with weight 1/k, and y = 0."""
    syn, dev = tiny
    x = np.zeros((3, syn.cfg.hidden), dtype=np.float32)
    g = run(dev, x, "f32")
    k = syn.cfg.top_k
    assert g["ids"].tolist() == [list(range(k))] * 3
    assert np.all(g["w"] == np.float32(1.0 / k))
    assert np.all(g["y"] == 0)


def test_sign_flip_of_down_codes_negates_y(tiny):
    syn, dev = tiny

    def flip(experts):
        for e in experts:
            experts[e]["codes_d"] = experts[e]["codes_d"] ^ np.uint8(0x80)
    _, devf = tiny_variant(syn, mutate=flip)
    x = syn.x(n=5, stream=4)
    a = run(dev, x, "f32")
    b = run(devf, x, "f32")
    assert np.array_equal(a["ids"], b["ids"])
    # The decoded down weights are negated exactly; the products are accumulated by
    # v_dot2_f32_f16, whose fp32 rounding is not sign-symmetric, so the negation holds
    # to fp32 rounding rather than bit for bit.
    scale = np.abs(a["y"]).max(axis=1, keepdims=True)
    assert np.all(np.abs(b["y"] + a["y"]) <= 2.0 ** -20 * scale)


@pytest.mark.parametrize("T", [1, 5])
def test_top1_routing(tiny, T):
    """k = 1: every routing weight is 1 and y is the selected expert's output."""
    syn, _ = tiny
    v, dev = tiny_variant(syn, top_k=1)
    x = syn.x(n=T, stream=70 + T)
    g = run(dev, x, "f32")
    assert g["status"] == _lib.OK
    assert np.all(g["w"] == 1.0)
    compare(syn, x, "f32", g, 1)


def test_top1_routing_tiled_kernels(mini):
    """k = 1 on shapes that take the one-token FC2 and the matrix-core kernels."""
    syn, _ = mini
    v, dev = tiny_variant(syn, top_k=1)
    for T in (1, 40):
        x = syn.x(n=T, stream=80 + T)
        g = run(dev, x, "bf16")
        assert g["status"] == _lib.OK
        compare(syn, x, "bf16", g, 1)


def test_k_equals_E_gives_full_softmax(tiny):
    syn, _ = tiny
    E = syn.cfg.n_experts
    _, dev = tiny_variant(syn, top_k=E)
    x = syn.x(n=3, stream=5)
    g = run(dev, x, "f32")
    x64 = oracle.x_value(x, "f32")
    lg = oracle.router_logits(syn.router_w, x64)
    p = oracle.softmax(lg)
    for t in range(3):
        assert sorted(g["ids"][t].tolist()) == list(range(E))
        np.testing.assert_allclose(g["w"][t], p[t][g["ids"][t]], atol=1e-5)
    compare(syn, x, "f32", g, E)


def test_mixed_formats_tiny(tiny):
    syn, _ = tiny
    fm = [synth.FMT_MXFP4 if e % 2 else synth.FMT_VQ2 for e in range(syn.cfg.n_experts)]
    v, dev = tiny_variant(syn, formats=fm)
    x = syn.x(n=8, stream=6)
    g = run(dev, x, "f32")
    assert g["status"] == _lib.OK
    compare(v, x, "f32", g, syn.cfg.top_k)


def test_absent_expert_is_reported_and_left_out(tiny):
    syn, _ = tiny
    x = syn.x()
    x64 = oracle.x_value(x, "f32")
    ids = oracle.topk(oracle.router_logits(syn.router_w, x64), syn.cfg.top_k)
    gone = int(np.bincount(ids.reshape(-1)).argmax())
    fm = list(syn.formats)
    fm[gone] = synth.FMT_ABSENT
    v, dev = tiny_variant(syn, formats=fm)
    g = run(dev, x, "f32")
    assert g["status"] == _lib.ENOTRESIDENT and g["info"] == gone
    r = oracle.forward(syn, x64, syn.cfg.top_k, forced_selection=g["ids"])
    keep = (g["ids"] != gone)[:, :, None]
    y_ref = (r["w"][:, :, None] * r["o"] * keep).sum(axis=1)
    err = np.abs(g["y"] - y_ref).max(axis=1) / np.abs(y_ref).max(axis=1)
    assert err.max() <= 1e-2


def test_one_token_absent_experts_reported(tiny):
    """One-token steps take their own worklist kernel: two selected experts absent, the
    lowest one reported, both left out of y."""
    syn, _ = tiny
    x = syn.x()[:1]
    x64 = oracle.x_value(x, "f32")
    ids = oracle.topk(oracle.router_logits(syn.router_w, x64), syn.cfg.top_k)[0]
    fm = list(syn.formats)
    for e in ids:
        fm[int(e)] = synth.FMT_ABSENT
    v, dev = tiny_variant(syn, formats=fm)
    g = run(dev, x, "f32")
    assert g["status"] == _lib.ENOTRESIDENT and g["info"] == int(min(ids))
    assert np.array_equal(g["ids"][0], ids)
    assert np.all(g["y"] == 0.0)  # every routed expert absent: nothing is added
    # one of the two absent: y is the other expert's weighted output
    fm = list(syn.formats)
    fm[int(ids[1])] = synth.FMT_ABSENT
    v, dev = tiny_variant(syn, formats=fm)
    g = run(dev, x, "f32")
    assert g["status"] == _lib.ENOTRESIDENT and g["info"] == int(ids[1])
    r = oracle.forward(syn, x64, syn.cfg.top_k, forced_selection=g["ids"])
    y_ref = r["w"][0, 0] * r["o"][0, 0]
    err = np.abs(g["y"][0] - y_ref).max() / np.abs(y_ref).max()
    assert err <= 1e-2


def test_slot_outside_pool_is_reported(tiny):
    syn, _ = tiny
    v, dev = tiny_variant(syn)
    offs = dev.slot_offsets.copy()
    x = syn.x()
    ids = oracle.topk(oracle.router_logits(syn.router_w, oracle.x_value(x, "f32")), syn.cfg.top_k)
    e = int(ids[0, 0])
    offs[e] = dev.pool_bytes - 256
    dev.set_slots(offs, dev.formats)
    g = run(dev, x, "f32")
    assert g["status"] == _lib.ENOTRESIDENT and g["info"] == e
    offs[e] = 128  # misaligned
    dev.set_slots(offs, dev.formats)
    g = run(dev, x, "f32")
    assert g["status"] == _lib.ENOTRESIDENT


# ---------------------------------------------------------------------------------
# The largest expert count and top-k the library takes (1024 experts, top-32), on a
# narrow layer: the one-token worklist, the fused and the separate top-k, the
# matrix-core router from 64 tokens on, and prefill
# ---------------------------------------------------------------------------------

MAXE = synth.Config("maxe", 5, 128, 128, 1024, 32, "bf16", "normal", seed=9191)


@pytest.fixture(scope="module")
def maxe():
    syn = synth.SynthLayer(MAXE)
    return syn, DeviceLayer.from_synth(syn)


@pytest.mark.parametrize("T", [1, 5, 40, 80])
def test_max_experts_and_top_k(maxe, T):
    syn, dev = maxe
    x = syn.x(n=T, stream=130 + T)
    say(f"maxe step T={T}")
    g = run(dev, x, "bf16")
    assert g["status"] == _lib.OK
    compare(syn, x, "bf16", g, MAXE.top_k)
    info = g["step"].info(T)
    assert info["n_pairs"] == T * MAXE.top_k
    assert info["experts"] == sorted(set(g["ids"].reshape(-1).tolist()))


def test_max_experts_and_top_k_mixed_formats_and_prefill(maxe):
    syn, _ = maxe
    fm = [synth.FMT_MXFP4 if e % 5 == 0 else synth.FMT_VQ2 for e in range(MAXE.n_experts)]
    v, dev = tiny_variant(syn, formats=fm)
    x = syn.x(n=70, stream=150)
    say("maxe mixed T=70")
    g = run(dev, x, "bf16")
    assert g["status"] == _lib.OK
    compare(v, x, "bf16", g, MAXE.top_k)
    say("maxe mixed prefill T=70")
    gp = run_prefill(dev, x, "bf16")
    assert gp["status"] == _lib.OK
    compare(v, x, "bf16", gp, MAXE.top_k, check_h=False)


# ---------------------------------------------------------------------------------
# A mid-size layer whose shapes take the tiled FC kernels (K a multiple of 1024)
# ---------------------------------------------------------------------------------

MINI = synth.Config("mini", 6, 2048, 1024, 16, 4, "bf16", "normal", seed=4242)


@pytest.fixture(scope="module")
def mini():
    syn = synth.SynthLayer(MINI)
    return syn, DeviceLayer.from_synth(syn)


@pytest.mark.parametrize("T", [1, 2, 5, 17, 64, 100])
def test_mini_tiled_kernels(mini, T):
    syn, dev = mini
    x = syn.x(n=T, stream=20 + T)
    say(f"mini step T={T}")
    g = run(dev, x, "bf16")
    assert g["status"] == _lib.OK
    compare(syn, x, "bf16", g, MINI.top_k)


def test_mini_mixed_formats(mini):
    syn, _ = mini
    fm = [synth.FMT_MXFP4 if e % 3 == 0 else synth.FMT_VQ2 for e in range(MINI.n_experts)]
    v, dev = tiny_variant(syn, formats=fm)
    for T in (1, 9):
        x = syn.x(n=T, stream=40 + T)
        g = run(dev, x, "bf16")
        assert g["status"] == _lib.OK
        compare(v, x, "bf16", g, MINI.top_k)


def test_mini_one_token_absent_expert(mini):
    """One token at K = 1024 (the one-token FC2 kernel): a selected expert absent is
    reported and its contribution left out, the other three added."""
    syn, _ = mini
    x = syn.x(n=1, stream=77)
    x64 = oracle.x_value(x, "bf16")
    ids = oracle.topk(oracle.router_logits(syn.router_w, x64), MINI.top_k)[0]
    gone = int(ids[2])
    fm = list(syn.formats)
    fm[gone] = synth.FMT_ABSENT
    v, dev = tiny_variant(syn, formats=fm)
    g = run(dev, x, "bf16")
    assert g["status"] == _lib.ENOTRESIDENT and g["info"] == gone
    r = oracle.forward(syn, x64, MINI.top_k, forced_selection=g["ids"])
    keep = (g["ids"] != gone)[:, :, None]
    y_ref = (r["w"][:, :, None] * r["o"] * keep).sum(axis=1)
    err = np.abs(g["y"] - y_ref).max(axis=1) / np.abs(y_ref).max(axis=1)
    assert err.max() <= 1e-2


def test_mini_fp32_activations(mini):
    syn, dev = mini
    x = oracle.x_value(syn.x(n=3, stream=50), "bf16").astype(np.float32) * np.float32(1.37)
    g = run(dev, x, "f32")
    compare(syn, x, "f32", g, MINI.top_k)


# ---------------------------------------------------------------------------------
# Full-width experts with few of them: every expert takes more than one 16-token group
# ---------------------------------------------------------------------------------

WIDE = synth.Config("wide", 40, 7168, 2048, 4, 2, "bf16", "normal", seed=4343)


def test_wide_fp32_activations_decode_and_prefill():
    # fp32 x at the full hidden size (seven 1024-column slices, each with its own
    # power-of-two factor when staged): the fp32 router, the one-token and the matrix-core
    # FC1 at K = 7168, and prefill's fp32 staging.  x = bf16 values times 1.37, so the
    # values are not bf16.
    syn = synth.SynthLayer(WIDE, cache=False)
    dev = DeviceLayer.from_synth(syn)
    for T in (1, 17, 40):
        x = oracle.x_value(syn.x(n=T, stream=160 + T), "bf16").astype(np.float32) * np.float32(1.37)
        say(f"wide fp32 T={T}")
        g = run(dev, x, "f32")
        assert g["status"] == _lib.OK
        compare(syn, x, "f32", g, WIDE.top_k)
        if T == 40:
            say("wide fp32 prefill T=40")
            gp = run_prefill(dev, x, "f32")
            assert gp["status"] == _lib.OK
            compare(syn, x, "f32", gp, WIDE.top_k, check_h=False)
    del dev
    torch.cuda.empty_cache()


def test_wide_experts_split_into_token_groups():
    syn = synth.SynthLayer(WIDE, cache=False)
    dev = DeviceLayer.from_synth(syn)
    for T in (40, 17):
        x = syn.x(n=T, stream=60 + T)
        say(f"wide step T={T}")
        g = run(dev, x, "bf16")
        assert g["status"] == _lib.OK
        counts = np.bincount(g["ids"].ravel(), minlength=WIDE.n_experts)
        if T == 40:
            assert counts.max() > 16  # 80 pairs over 4 experts: some group is full and split
        compare(syn, x, "bf16", g, WIDE.top_k)
    # the same with two experts in MXFP4: the format changes between token groups
    v, dev = tiny_variant(syn, formats=[synth.FMT_MXFP4, synth.FMT_VQ2, synth.FMT_MXFP4, synth.FMT_VQ2])
    x = syn.x(n=40, stream=99)
    say("wide step T=40, mixed formats")
    g = run(dev, x, "bf16")
    assert g["status"] == _lib.OK
    compare(v, x, "bf16", g, WIDE.top_k)
    # one-token steps (their own FC2 kernel, K = 2048, six of its eight expert waves idle)
    chosen = set()
    for st in range(100, 104):
        x = syn.x(n=1, stream=st)
        say(f"wide step T=1 stream {st}, mixed formats")
        g = run(dev, x, "bf16")
        assert g["status"] == _lib.OK
        compare(v, x, "bf16", g, WIDE.top_k)
        chosen |= set(int(e) for e in g["ids"].ravel())
    assert chosen & {0, 2} and chosen & {1, 3}  # both formats went through it


# ---------------------------------------------------------------------------------
# Full-size layers (H=7168, I=2048, E=256, k=8), sampled tokens
# ---------------------------------------------------------------------------------

def _full(name):
    cfg = synth.PRESETS[name]
    syn_dev = synth.SynthLayer(cfg, cache=False)
    say(f"building {name} pool")
    dev = DeviceLayer.from_synth(syn_dev)
    return synth.SynthLayer(cfg), dev


@pytest.fixture(scope="module")
def b1():
    syn, dev = _full("b1")
    yield syn, dev
    del dev
    torch.cuda.empty_cache()


def test_b1_decode_sampled_rows(b1):
    syn, dev = b1
    say("b1 decode")
    _check_decode(syn, dev, [int(np.nonzero(syn.formats == synth.FMT_VQ2)[0][5])], rows=slice(0, 2048, 97))


def test_b1_steps(b1):
    syn, dev = b1
    st = Step(dev, 1)
    for s in range(2):
        x = syn.x(n=1, stream=100 + s)
        say(f"b1 token {s}")
        g = run(dev, x, "bf16", step=st)
        assert g["status"] == _lib.OK
        info = st.info(1)
        assert info["n_active"] == 8 and info["experts"] == sorted(g["ids"][0].tolist())
        res = compare(syn, x, "bf16", g, 8)
        say("b1", {k: v for k, v in res.items() if k != "ref"})


@pytest.fixture(scope="module")
def b32():
    syn, dev = _full("b32")
    yield syn, dev
    del dev
    torch.cuda.empty_cache()


def test_b32_step(b32):
    syn, dev = b32
    x = syn.x()
    say("b32 step")
    g = run(dev, x, "bf16")
    assert g["status"] == _lib.OK
    info = g["step"].info(32)
    uniq = sorted(set(g["ids"].reshape(-1).tolist()))
    assert info["experts"] == uniq and info["n_pairs"] == 256
    say("b32 unique experts", len(uniq))
    res = compare(syn, x, "bf16", g, 8)  # every token
    say("b32", {k: v for k, v in res.items() if k != "ref"})


@pytest.fixture(scope="module")
def b8mx():
    syn, dev = _full("b8mx")
    yield syn, dev
    del dev
    torch.cuda.empty_cache()


def test_b8mx_decode_sampled_rows_mxfp4(b8mx):
    """Full-size MXFP4 expert (one of the 52 most popular): sampled rows bit for bit."""
    syn, dev = b8mx
    say("b8mx decode")
    _check_decode(syn, dev, [int(np.nonzero(syn.formats == synth.FMT_MXFP4)[0][3])], rows=slice(0, 2048, 97))


def test_b8mx_step(b8mx):
    syn, dev = b8mx
    x = syn.x()
    say("b8mx step")
    g = run(dev, x, "bf16")
    assert g["status"] == _lib.OK
    ids = g["ids"]
    mx = np.nonzero(syn.formats == synth.FMT_MXFP4)[0]
    n_mx = int(np.isin(np.unique(ids), mx).sum())
    say("b8mx unique", len(np.unique(ids)), "mxfp4", n_mx)
    assert n_mx > 0
    assert np.isin(ids, mx).any(axis=1).sum() >= 4, "most tokens should reach an MXFP4 expert"
    res = compare(syn, x, "bf16", g, 8)  # every token
    say("b8mx", {k: v for k, v in res.items() if k != "ref"})


# ---------------------------------------------------------------------------------
# moe_vq_forward: the whole step in one call, bit for bit the three calls
# ---------------------------------------------------------------------------------

@pytest.mark.parametrize("T", [1, 5, 40])
def test_forward_call_matches_three_calls(mini, T):
    syn, dev = mini
    x = syn.x(n=T, stream=500 + T)
    g = run(dev, x, "bf16")
    st = Step(dev, T)
    from gpu_util import x_tensor
    y = st.step(x_tensor(x, "bf16")).cpu().numpy().astype(np.float64)
    assert st.check()[0] == _lib.OK
    assert np.array_equal(st.ids[:T].cpu().numpy(), g["ids"])
    assert np.array_equal(st.w[:T].cpu().numpy().astype(np.float64), g["w"])
    assert np.array_equal(y, g["y"])
    assert np.array_equal(st.h[:T * MINI.top_k].cpu().numpy().astype(np.float64).reshape(g["h"].shape), g["h"])
