"""Pins of the fp64 oracle against what the format and the mathematics fix.

Nothing here compares the oracle with itself re-typed: each test checks an
invariant of the format (sign symmetry, lossless round trip, group structure), a
closed form, a special case that reduces to a simpler computation, a published
table (OCP MX v1.0 E2M1 values), or a scalar brute force written independently
of the vectorised code.
"""
import copy
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


class ArrLayer:
    def __init__(self, codebook, router_w, experts):
        self.codebook = codebook
        self.router_w = router_w
        self._experts = experts

    def expert(self, e):
        return self._experts[e]


@pytest.fixture(scope="module")
def tiny():
    return synth.SynthLayer(synth.PRESETS["tiny"])


def tiny_arrays(layer):
    cfg = layer.cfg
    return ArrLayer(layer.codebook.copy(), layer.router_w.copy(),
                    [copy.deepcopy(layer.expert(e)) for e in range(cfg.n_experts)])


# ---------------------------------------------------------------------------------
# O1: VQ2 decode
# ---------------------------------------------------------------------------------

@pytest.mark.parametrize("scale", [0.005, 0.0137, 0.02, 1.0, 6.0e-8, 65504.0, 0.0])
def test_vq2_sign_symmetry_exhaustive(tiny, scale):
    """decode(b ^ 0x80) == -decode(b) bitwise for all 256 words, and the 256 signed
    codewords sum to exactly zero (the codebook is sign-symmetric)."""
    codes = np.arange(256, dtype=np.uint8).reshape(2, 128)      # 2 rows x 128 words
    flipped = codes ^ np.uint8(0x80)
    scales = np.full((2, 4), scale, dtype=np.float16)           # 512 weights / row
    a = oracle.vq2_decode(codes, scales, tiny.codebook)
    b = oracle.vq2_decode(flipped, scales, tiny.codebook)
    assert np.array_equal(a.view(np.uint64), (-b).view(np.uint64))
    total = a.reshape(-1, 4).sum(axis=0)
    assert np.all(total == 0.0)


def test_vq2_round_trip_exhaustive_tiny(tiny):
    """Lossless round trip: W / s is exactly a signed codeword, and the nearest
    signed codeword (ties -> lowest word) recovers every stored word."""
    for e in range(tiny.cfg.n_experts):
        ex = tiny.expert(e)
        for m in "gud":
            W = oracle.vq2_decode(ex["codes_" + m], ex["scales_" + m], tiny.codebook)
            s = np.repeat(ex["scales_" + m].astype(np.float64), 128, axis=1)
            assert np.all(s > 0)
            back = oracle.vq2_encode_nearest(W / s, tiny.codebook)
            assert np.array_equal(back, ex["codes_" + m])


def test_vq2_round_trip_sampled_full_size():
    cfg = synth.PRESETS["b1"]
    cb = synth.draw_codebook(cfg.seed)
    ex = synth.draw_expert(cfg, 7, synth.FMT_VQ2)
    rows = [0, 1, 777, 2047]
    for m, nrows in (("g", 2048), ("d", 7168)):
        rr = [r for r in rows if r < nrows]
        W = oracle.vq2_decode(ex["codes_" + m][rr], ex["scales_" + m][rr], cb)
        s = np.repeat(ex["scales_" + m][rr].astype(np.float64), 128, axis=1)
        back = oracle.vq2_encode_nearest(W / s, cb)
        assert np.array_equal(back, ex["codes_" + m][rr])


def test_vq2_constant_row_closed_form(tiny):
    """All words of row n equal b, scale s, x = 1  =>  g_n = s * sgn(b) * (H/4) * sum_d CB[b & 0x7F, d]."""
    H, I = 256, 4
    cb = tiny.codebook
    for b in (0, 5, 127, 128, 200, 255):
        codes = np.full((I, H // 4), b, dtype=np.uint8)
        scales = np.full((I, H // 128), 0.0137, dtype=np.float16)
        W = oracle.vq2_decode(codes, scales, cb)
        r = oracle.expert_mlp(W, W, np.zeros((H, I)), np.ones((1, H)))
        s = float(np.float16(0.0137))
        sgn = -1.0 if b & 0x80 else 1.0
        comp = [float(v) for v in cb[b & 0x7F]]
        expected = s * sgn * (H // 4) * (comp[0] + comp[1] + comp[2] + comp[3])
        assert r["g"].shape == (1, I)
        np.testing.assert_allclose(r["g"][0], expected, rtol=1e-14, atol=0)


def test_vq2_scale_group_structure(tiny):
    """A single nonzero scale (row n, group q) makes exactly the weights of row n,
    columns [128q, 128q + 128) nonzero (the codebook has no zero vector, but single
    components may be zero, so compare with the support of the codewords)."""
    H, I = 512, 3
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 256, (I, H // 4), dtype=np.uint8)
    support = np.abs(oracle.signed_codebook(tiny.codebook))[codes].reshape(I, H) != 0
    for n in range(I):
        for q in range(H // 128):
            scales = np.zeros((I, H // 128), dtype=np.float16)
            scales[n, q] = 0.5
            W = oracle.vq2_decode(codes, scales, tiny.codebook)
            mask = np.zeros((I, H), dtype=bool)
            mask[n, 128 * q:128 * (q + 1)] = True
            assert np.array_equal(W != 0, mask & support)


def test_vq2_decode_matches_scalar_reading(tiny):
    """The vectorised decode equals a scalar reading of the words (independent index
    arithmetic) for every weight of one tiny expert."""
    ex = tiny.expert(3)
    for m in "gud":
        W = oracle.vq2_decode(ex["codes_" + m], ex["scales_" + m], tiny.codebook)
        rows, cols = W.shape
        for n in range(rows):
            for k in range(cols):
                assert W[n, k] == oracle.moe_vq_oracle._scalar_weight(ex, tiny.codebook, m, n, k)


# ---------------------------------------------------------------------------------
# O1': MXFP4 decode
# ---------------------------------------------------------------------------------

def _golden_e2m1():
    vals = {}
    with open(os.path.join(GOLDEN, "e2m1_ocp_mx_v1.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            code, v = line.split()
            vals[int(code, 2)] = float(v)
    assert len(vals) == 16
    return vals


def test_e2m1_table_matches_ocp_spec():
    g = _golden_e2m1()
    for q in range(16):
        v = float(oracle.e2m1_value(np.array([q]))[0])
        assert v == g[q] and math.copysign(1, v) == math.copysign(1, g[q])


@pytest.mark.parametrize("e", [118, 119, 120, 127, 1, 254])
def test_mxfp4_decode_exhaustive(e):
    """All 256 bytes x E8M0 exponent e: value = golden E2M1 * 2^(e-127), low nibble
    first; flipping bit 3 of a nibble negates its weight."""
    g = _golden_e2m1()
    nib = np.arange(256, dtype=np.uint8).reshape(8, 32)             # 8 rows x 64 weights
    e8 = np.full((8, 2), e, dtype=np.uint8)
    W = oracle.mxfp4_decode(nib, e8)
    for r in range(8):
        for j in range(32):
            byte = int(nib[r, j])
            assert W[r, 2 * j] == g[byte & 0xF] * 2.0 ** (e - 127)
            assert W[r, 2 * j + 1] == g[byte >> 4] * 2.0 ** (e - 127)
    Wf = oracle.mxfp4_decode(nib ^ np.uint8(0x88), e8)
    assert np.array_equal(Wf, -W)


def test_mxfp4_worked_byte():
    """Byte 0x21 with exponent 127: weight 0 (low nibble 1) = 0.5, weight 1 (high nibble 2) = 1.0."""
    W = oracle.mxfp4_decode(np.array([[0x21] * 16], dtype=np.uint8), np.array([[127]], dtype=np.uint8))
    assert W[0, 0] == 0.5 and W[0, 1] == 1.0
    assert np.isnan(oracle.e8m0_value(np.array([255]))[0])


# ---------------------------------------------------------------------------------
# O2..O5: routing
# ---------------------------------------------------------------------------------

def test_router_zero_and_one_hot(tiny):
    H = tiny.cfg.hidden
    assert np.all(oracle.router_logits(tiny.router_w, np.zeros((2, H))) == 0)
    x = np.zeros((3, H))
    cols = [0, 17, H - 1]
    for t, j in enumerate(cols):
        x[t, j] = 1.0
    lg = oracle.router_logits(tiny.router_w, x)
    rw = synth.bf16_bits_to_f32(tiny.router_w).astype(np.float64)
    for t, j in enumerate(cols):
        assert np.array_equal(lg[t], rw[:, j])


def test_router_matches_scalar_loop(tiny):
    x = oracle.x_value(tiny.x(), "f32")
    lg = oracle.router_logits(tiny.router_w, x)
    rw = tiny.router_w
    for t in range(x.shape[0]):
        for e in range(tiny.cfg.n_experts):
            ref = math.fsum(float(synth.bf16_bits_to_f32(rw[e, j:j + 1])[0]) * float(x[t, j])
                            for j in range(x.shape[1]))
            assert abs(lg[t, e] - ref) <= 1e-13 * (1 + abs(ref))


def test_softmax_closed_form():
    lg = np.log(np.array([[1.0, 2.0, 3.0, 6.0]]))
    p = oracle.softmax(lg)
    np.testing.assert_allclose(p[0], [1 / 12, 2 / 12, 3 / 12, 6 / 12], rtol=1e-15)
    # shift invariance
    np.testing.assert_allclose(oracle.softmax(lg + 1234.5), p, rtol=1e-12)


def test_silu_closed_forms():
    g = np.array([0.0, 1.0, -1.0, 40.0, -40.0])
    s = oracle.silu(g)
    assert s[0] == 0.0
    assert abs(s[1] - 0.7310585786300049) < 1e-16
    assert abs(s[2] + 0.2689414213699951) < 1e-16
    assert abs(s[3] - 40.0) < 1e-15
    assert abs(s[4]) < 1e-15
    z = np.linspace(-8, 8, 33)
    np.testing.assert_allclose(oracle.silu(-z), oracle.silu(z) - z, atol=1e-14)


def test_routing_weights_sum_to_one():
    for name in ("tiny", "b1"):
        cfg = synth.PRESETS[name]
        rw = synth.draw_router(cfg)
        x = oracle.x_value(synth.draw_x(cfg, n=16, router_bits=rw), cfg.x_dtype)
        _, ids, w = oracle.route(rw, x, cfg.top_k)
        assert np.all(np.abs(w.sum(axis=1) - 1.0) <= 1e-14)
        assert np.all(w > 0)
        for row in ids:
            assert len(set(row.tolist())) == cfg.top_k


def test_topk_equals_full_softmax_when_k_is_E(tiny):
    """SC2: k = E  =>  w equals the full softmax p (in descending logit order)."""
    x = oracle.x_value(tiny.x(), "f32")
    lg, ids, w = oracle.route(tiny.router_w, x, tiny.cfg.n_experts)
    p = oracle.softmax(lg)
    np.testing.assert_allclose(w, np.take_along_axis(p, ids, axis=1), rtol=1e-14)
    assert np.all(np.diff(np.take_along_axis(lg, ids, axis=1), axis=1) <= 0)


def test_topk_matches_bruteforce():
    rng = np.random.default_rng(11)
    cases = [rng.standard_normal(8) for _ in range(20)]
    cases += [np.array([1.0, 2.0, 2.0, 0.5, 2.0, -1.0, 0.0, 2.0]),   # 4-way tie at the top
              np.zeros(8),                                             # all tied
              np.array([3.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0])]
    for lg in cases:
        for k in (1, 2, 3, 8):
            assert oracle.topk(lg[None, :], k)[0].tolist() == oracle.topk_bruteforce(lg, k)


def test_zero_input_selects_lowest_ids(tiny):
    """SC5: x = 0 => all logits tie => S = {0..k-1}, w = 1/k, y = 0."""
    k = tiny.cfg.top_k
    r = oracle.forward(tiny, np.zeros((2, tiny.cfg.hidden)), k)
    assert r["ids"].tolist() == [list(range(k))] * 2
    assert np.all(r["w"] == 1.0 / k)
    assert np.all(r["y"] == 0)


# ---------------------------------------------------------------------------------
# O6..O8 and the whole step
# ---------------------------------------------------------------------------------

def test_forward_matches_dense_bruteforce(tiny):
    """Scalar brute force of the dense all-expert form equals the sparse oracle."""
    x = oracle.x_value(tiny.x(), "f32")
    r = oracle.forward(tiny, x, tiny.cfg.top_k)
    yb = oracle.forward_bruteforce(tiny, x, tiny.cfg.top_k)
    scale = np.abs(yb).max()
    assert np.abs(r["y"] - yb).max() <= 1e-12 * scale


def test_single_expert_is_plain_swiglu_mlp(tiny):
    """SC1: E = 1, k = 1  =>  w = 1 and y is a plain SwiGLU MLP of the decoded weights."""
    lay = ArrLayer(tiny.codebook, tiny.router_w[:1].copy(), [tiny.expert(0)])
    x = oracle.x_value(tiny.x(), "f32")[:2]
    r = oracle.forward(lay, x, 1)
    assert np.all(r["w"] == 1.0) and np.all(r["ids"] == 0)
    yb = oracle.forward_bruteforce(lay, x, 1)
    assert np.abs(r["y"] - yb).max() <= 1e-12 * np.abs(yb).max()


@pytest.mark.parametrize("mat", ["u", "d"])
def test_sign_flip_negates_output_exactly(tiny, mat):
    """SC4: flipping the sign bit of every W_u (or W_d) word negates y exactly."""
    lay = tiny_arrays(tiny)
    x = oracle.x_value(tiny.x(), "f32")
    y0 = oracle.forward(lay, x, 2)["y"]
    for e in range(tiny.cfg.n_experts):
        lay._experts[e]["codes_" + mat] = lay._experts[e]["codes_" + mat] ^ np.uint8(0x80)
    y1 = oracle.forward(lay, x, 2)["y"]
    assert np.array_equal(y1, -y0)


def test_zero_scale_group_contributes_nothing(tiny):
    """SC6: zeroing group q's scales in W_g and W_u equals zeroing x's columns of group q
    for the expert outputs."""
    lay = tiny_arrays(tiny)
    x = oracle.x_value(tiny.x(), "f32")
    q = 1
    for e in range(tiny.cfg.n_experts):
        for m in "gu":
            lay._experts[e]["scales_" + m][:, q] = 0
    xz = x.copy()
    xz[:, 128 * q:128 * (q + 1)] = 0
    ids = oracle.forward(tiny, x, 2)["ids"]
    # the routing weights see x, so compare the per-pair expert outputs h and o
    a = oracle.forward(lay, x, 2, forced_selection=ids)
    b = oracle.forward(tiny, xz, 2, forced_selection=ids)
    for key in ("h", "o"):
        np.testing.assert_allclose(a[key], b[key], rtol=1e-13, atol=1e-15 * np.abs(b[key]).max())
    assert np.abs(a["h"] - oracle.forward(tiny, x, 2)["h"]).max() > 0


def test_one_hot_input_reads_a_column(tiny):
    """SC7: x = e_j  =>  g_n = W_g[n, j] (a decode check through the product)."""
    ex = tiny.expert(5)
    Wg, Wu, Wd = oracle.decode_expert(ex, tiny.codebook)
    for j in (0, 1, 127, 128, 255):
        x = np.zeros((1, 256))
        x[0, j] = 1.0
        g = oracle.expert_mlp(Wg, Wu, Wd, x)["g"][0]
        for n in range(0, 128, 13):
            assert g[n] == oracle.moe_vq_oracle._scalar_weight(ex, tiny.codebook, "g", n, j)


def test_forced_selection_renormalises(tiny):
    x = oracle.x_value(tiny.x(), "f32")
    forced = np.array([[7, 0], [1, 2], [3, 4], [5, 6]])
    r = oracle.forward(tiny, x, 2, forced_selection=forced)
    p = oracle.softmax(r["logits"])
    sel = np.take_along_axis(p, forced, axis=1)
    np.testing.assert_allclose(r["w"], sel / sel.sum(1, keepdims=True), rtol=1e-15)


# ---------------------------------------------------------------------------------
# Near-tie acceptance
# ---------------------------------------------------------------------------------

def test_selection_validity_rule():
    lg = np.array([[3.0, 2.0, 2.0 + 1e-9, 0.0]])
    delta = np.full_like(lg, 1e-8)
    assert oracle.selection_is_valid(np.array([[0, 2]]), lg, delta, 2)
    assert oracle.selection_is_valid(np.array([[0, 1]]), lg, delta, 2)      # within the bound
    assert not oracle.selection_is_valid(np.array([[0, 3]]), lg, delta, 2)
    assert not oracle.selection_is_valid(np.array([[0, 0]]), lg, delta, 2)
    assert not oracle.selection_is_valid(np.array([[2, 0]]), lg, delta, 2)  # wrong order
    tight = np.zeros_like(lg)
    assert not oracle.selection_is_valid(np.array([[0, 1]]), lg, tight, 2)


def test_fp32_bound_covers_fp32_dot(tiny):
    """The error bound dominates the actual fp32 error of a fp32 dot product."""
    cfg = synth.PRESETS["b1"]
    rw = synth.draw_router(cfg)
    x = oracle.x_value(synth.draw_x(cfg, n=4, router_bits=rw), "bf16")
    exact = oracle.router_logits(rw, x)
    f32 = (x.astype(np.float32) @ synth.bf16_bits_to_f32(rw).T).astype(np.float64)
    assert np.all(np.abs(f32 - exact) <= oracle.fp32_dot_error_bound(rw, x))


# ---------------------------------------------------------------------------------
# O6' SwiGLU clamp and O9 shared expert (readings R14 and R13)
# ---------------------------------------------------------------------------------

def _gate_up_extent(lay, x):
    """max |g| and max |u| over every expert and token of the tiny layer."""
    m = 0.0
    for e in range(lay_experts(lay)):
        Wg, Wu, Wd = oracle.decode_expert(lay.expert(e), lay.codebook)
        r = oracle.expert_mlp(Wg, Wu, Wd, x)
        m = max(m, float(np.abs(r["g"]).max()), float(np.abs(r["u"]).max()))
    return m


def lay_experts(lay):
    return lay.cfg.n_experts if hasattr(lay, "cfg") else len(lay._experts)


def test_clamp_leaves_values_inside_the_limit_alone(tiny):
    """With L above every |g| and |u| of the batch the clamp changes nothing, bit for bit;
    just below the largest it does."""
    x = oracle.x_value(tiny.x(), "f32")
    m = _gate_up_extent(tiny, x)
    y0 = oracle.forward(tiny, x, 2)["y"]
    assert np.array_equal(oracle.forward(tiny, x, 2, swiglu_limit=m * (1 + 1e-9))["y"], y0)
    assert not np.array_equal(oracle.forward(tiny, x, 2, swiglu_limit=m * 0.999)["y"], y0)


def test_clamp_form_gate_one_sided_up_two_sided():
    """R14's form: the gate is only capped from above (a very negative gate keeps its
    value), the up projection is clamped on both sides."""
    L = 1.5
    g = np.array([-10.0, -1.0, 0.5, 3.0, 3.0, -10.0])
    u = np.array([1.0, -4.0, 0.25, 2.0, -7.0, 9.0])
    h = oracle.swiglu(g, u, L)
    sig = lambda v: 1.0 / (1.0 + math.exp(-v))
    want = [-10.0 * sig(-10.0) * 1.0, -1.0 * sig(-1.0) * -1.5, 0.5 * sig(0.5) * 0.25,
            1.5 * sig(1.5) * 1.5, 1.5 * sig(1.5) * -1.5, -10.0 * sig(-10.0) * 1.5]
    np.testing.assert_allclose(h, want, rtol=1e-15)
    assert np.isnan(oracle.swiglu(np.array([np.nan]), np.array([1.0]), L)[0])


def test_clamped_forward_matches_scalar_bruteforce(tiny):
    """With a limit that clamps a good share of g and u, the vectorised oracle equals the
    scalar brute force of the dense form."""
    x = oracle.x_value(tiny.x(), "f32")
    m = _gate_up_extent(tiny, x)
    L = 0.3 * m
    r = oracle.forward(tiny, x, tiny.cfg.top_k, swiglu_limit=L)
    yb = oracle.forward_bruteforce(tiny, x, tiny.cfg.top_k, swiglu_limit=L)
    assert np.abs(r["y"] - yb).max() <= 1e-12 * np.abs(yb).max()
    assert np.abs(r["y"] - oracle.forward(tiny, x, tiny.cfg.top_k)["y"]).max() > 1e-3 * np.abs(yb).max()


def test_shared_expert_alone_is_a_plain_swiglu_mlp(tiny):
    """O9 with every routed expert's down scales zeroed: y is the shared expert's MLP,
    equal to the one-expert layer of SC1 (brute force) built from the same arrays."""
    lay = tiny_arrays(tiny)
    for e in range(tiny.cfg.n_experts):
        lay._experts[e]["scales_d"][:] = 0
    shared = copy.deepcopy(tiny.expert(3))
    x = oracle.x_value(tiny.x(), "f32")
    r = oracle.forward(lay, x, 2, shared=shared)
    assert np.all(r["o"] == 0)
    one = ArrLayer(tiny.codebook, tiny.router_w[:1].copy(), [shared])
    yb = oracle.forward_bruteforce(one, x, 1)
    assert np.abs(r["y"] - yb).max() <= 1e-12 * np.abs(yb).max()
    assert np.array_equal(r["y"], r["o_shared"])


def test_shared_expert_matches_scalar_bruteforce(tiny):
    """Routed experts and the shared one (an MXFP4 expert), with the clamp: the sparse
    oracle equals the dense scalar brute force."""
    shared = synth.draw_expert(tiny.cfg, 99, synth.FMT_MXFP4)
    x = oracle.x_value(tiny.x(), "f32")[:2]
    L = 0.5 * _gate_up_extent(tiny, x)
    r = oracle.forward(tiny, x, 2, swiglu_limit=L, shared=shared)
    yb = oracle.forward_bruteforce(tiny, x, 2, swiglu_limit=L, shared=shared)
    assert np.abs(r["y"] - yb).max() <= 1e-12 * np.abs(yb).max()
    y_routed = oracle.forward(tiny, x, 2, swiglu_limit=L)["y"]
    np.testing.assert_allclose(r["y"] - y_routed, r["o_shared"], rtol=1e-12, atol=1e-14 * np.abs(yb).max())


# ---------------------------------------------------------------------------------
# O10: FP4 delta cache and confidence gate
# ---------------------------------------------------------------------------------

def _copies(layer, experts):
    """FP4 copies (the expert stored as MXFP4) for the given experts, None for the rest."""
    return lambda e: layer.expert_as(e, synth.FMT_MXFP4) if e in experts else None


def _tau_between_weights(w, q=0.5):
    """A gate value at quantile q of the routing weights, moved to the middle of the gap
    around it, so that no weight lies near it (any rounding of w takes the same side)."""
    s = np.unique(np.sort(w.reshape(-1)))
    i = int(np.clip(round(q * (len(s) - 1)), 0, len(s) - 2))
    assert s[i + 1] - s[i] > 1e-9
    return 0.5 * (s[i] + s[i + 1])


def test_gate_above_one_changes_nothing(tiny):
    """tau > 1: no renormalised weight reaches it, so every pair keeps its 2-bit expert."""
    x = oracle.x_value(tiny.x(), "f32")
    k = tiny.cfg.top_k
    r0 = oracle.forward(tiny, x, k)
    r1 = oracle.forward(tiny, x, k, fp4_copy=_copies(tiny, set(range(tiny.cfg.n_experts))), gate_tau=1.01)
    assert not r1["copy"].any()
    assert np.array_equal(r0["y"], r1["y"]) and np.array_equal(r0["h"], r1["h"])


def test_gate_zero_with_every_copy_is_the_fp4_layer(tiny):
    """tau = 0 and a copy of every expert: every pair takes its copy, so the step is the
    one of the layer whose experts are all stored in FP4 (same router, same selection)."""
    x = oracle.x_value(tiny.x(), "f32")
    k, E = tiny.cfg.top_k, tiny.cfg.n_experts
    lay4 = ArrLayer(tiny.codebook, tiny.router_w, [tiny.expert_as(e, synth.FMT_MXFP4) for e in range(E)])
    r = oracle.forward(tiny, x, k, fp4_copy=_copies(tiny, set(range(E))), gate_tau=0.0)
    r4 = oracle.forward(lay4, x, k)
    assert r["copy"].all()
    assert np.array_equal(r["y"], r4["y"]) and np.array_equal(r["h"], r4["h"])


@pytest.mark.parametrize("tau", [0.5, 0.6, 0.75])
def test_gate_at_one_half_or_more_passes_only_the_first_pair(tiny, tau):
    """The renormalised weights of a token sum to 1, so with tau >= 0.5 at most one pair
    passes, and it is the first (largest weight); it passes exactly when w_0 >= tau."""
    x = oracle.x_value(tiny.x(), "f32")
    k, E = tiny.cfg.top_k, tiny.cfg.n_experts
    r = oracle.forward(tiny, x, k, fp4_copy=_copies(tiny, set(range(E))), gate_tau=tau)
    assert not r["copy"][:, 1:].any()
    assert np.array_equal(r["copy"][:, 0], r["w"][:, 0] >= tau)


def test_copy_changes_only_the_gated_pairs(tiny):
    """Pairs that do not pass the gate (or whose expert has no copy) give the same h and o
    as without the delta cache; the gated ones give the copy's MLP (SC1 on the copy)."""
    x = oracle.x_value(tiny.x(), "f32")
    k, E = tiny.cfg.top_k, tiny.cfg.n_experts
    r0 = oracle.forward(tiny, x, k)
    tau = _tau_between_weights(r0["w"], 0.5)
    have = set(range(0, E, 2))
    r = oracle.forward(tiny, x, k, fp4_copy=_copies(tiny, have), gate_tau=tau)
    gated = r["copy"]
    assert gated.any() and (~gated).any()
    assert np.array_equal(gated, (r0["w"] >= tau) & np.isin(r0["ids"], list(have)))
    assert np.array_equal(r["h"][~gated], r0["h"][~gated]) and np.array_equal(r["o"][~gated], r0["o"][~gated])
    for t, i in zip(*np.nonzero(gated)):
        e = int(r["ids"][t, i])
        one = ArrLayer(tiny.codebook, tiny.router_w[:1].copy(), [tiny.expert_as(e, synth.FMT_MXFP4)])
        yb = oracle.forward_bruteforce(one, x[t:t + 1], 1)[0]
        assert np.abs(r["o"][t, i] - yb).max() <= 1e-12 * np.abs(yb).max()


def test_gated_forward_matches_scalar_bruteforce(tiny):
    """Copies for half the experts, tau inside the weight range: the sparse oracle equals
    the dense scalar brute force, which applies the gate on its own weights."""
    x = oracle.x_value(tiny.x(), "f32")[:4]
    k, E = tiny.cfg.top_k, tiny.cfg.n_experts
    r0 = oracle.forward(tiny, x, k)
    tau = _tau_between_weights(r0["w"], 0.5)
    above = r0["ids"][r0["w"] >= tau]
    cp = _copies(tiny, set(range(E)) - {int(above[0])})  # one gated expert without a copy
    r = oracle.forward(tiny, x, k, fp4_copy=cp, gate_tau=tau)
    yb = oracle.forward_bruteforce(tiny, x, k, fp4_copy=cp, gate_tau=tau)
    assert r["copy"].any() and (~r["copy"]).any()
    assert np.abs(r["y"] - yb).max() <= 1e-12 * np.abs(yb).max()
