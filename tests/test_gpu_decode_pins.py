"""Decode pinned through the GEMV on the GPU (the one-hot closed form).

With x = v * e_j (one token, one nonzero activation, v a power of two), FC1's gate and
up outputs are exactly v * W_g[:, j] and v * W_u[:, j]: one decoded weight per output,
no rounding in any summation order.  So every element of h = silu(g) * u must match the
oracle's decode to the rounding of SiLU's exponential, and one mis-decoded code byte,
sign or scale shows up as an O(1) error at the elements it feeds.  FC2 is pinned the
same way by handing moe_vq_fc2_combine a one-hot h: y[t] = sum_i w_i v_i W_d,i[:, j_i].
Each FC kernel family (one-token vector-ALU, matrix-core token groups, the generic
kernel, the one-token FC2 with its combine) is driven at the K it is built for, with
the hot column j spread over 1024-column slices, 128-wide scale groups, 16-byte chunks
and lone groups, in VQ2 and MXFP4.

The prefill form has no h output, so a layer is built whose up matrices are zero except
row n0 (zero scales; zero E2M1 codes): h is then one-hot at n0 and y isolates column n0
of W_d and the weights W_g[n0, j], W_u[n0, j].  Prefill rounds VQ2 weights to fp16 (2^-11)
and keeps h in bf16 (2^-9): 3.4e-3 of a term at most, checked at 5e-3 of the sum of the
terms' magnitudes.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from bit_vector_quantised_amd import _lib
from bit_vector_quantised_amd.layer import DeviceLayer, Step

from gpu_util import compare, run, run_prefill, say, x_tensor
from test_gpu_parity import tiny_variant

pytestmark = pytest.mark.gpu

# relative tolerance of one h element (hardware exponential in SiLU, one product)
H_TOL = 2e-6
# FC2: y element against the sum of its k terms' magnitudes (fp32 weight product and the
# k-term sum)
Y_TOL = 4e-6

LAYERS = {
    # name: (H, I, E, k) -- FC1 at K = H, FC2 at K = I
    "h2048_i1024": (2048, 1024, 16, 4),
    "h1024_i2048": (1024, 2048, 8, 2),
    "h7168_i2048": (7168, 2048, 4, 2),
    "h2048_i7168": (2048, 7168, 4, 2),
    "h256_i128": (256, 128, 8, 2),
    "h384_i640": (384, 640, 8, 2),
    "h2048_i1024_k12": (2048, 1024, 16, 12),
}


def make_layer(name, mixed=False, mutate=None, seed=5150):
    H, I, E, k = LAYERS[name]
    cfg = synth.Config(name, 4, H, I, E, k, "bf16", "normal", seed=seed)
    syn = synth.SynthLayer(cfg, cache=False)
    fm = [synth.FMT_MXFP4 if (mixed and e % 2 == 0) else synth.FMT_VQ2 for e in range(E)]
    return tiny_variant(syn, formats=fm, mutate=mutate)


class Decoded:
    """Per-expert fp64 weights from the oracle's decode, computed once."""

    def __init__(self, v):
        self.v, self.cache = v, {}

    def __call__(self, e):
        if e not in self.cache:
            self.cache[e] = oracle.decode_expert(self.v.expert(e), self.v.codebook)
        return self.cache[e]


def spread_columns(K, n, seed):
    """n columns over [0, K): the first and last of slices, scale groups and 16-byte
    chunks, the middle, and random ones."""
    fixed = [0, 1, 3, 4, 63, 64, 127, 128, 131, 255, 257, 511, 513, K // 2 + 5, K - 128, K - 65, K - 1]
    fixed += [s * 1024 + o for s in range(K // 1024) for o in (0, 1023) if s * 1024 + o < K]
    fixed = sorted({c for c in fixed if 0 <= c < K})
    rng = np.random.default_rng(seed)
    extra = rng.choice(K, size=max(0, n - len(fixed)), replace=False).tolist()
    cols = fixed + [c for c in extra if c not in fixed]
    rng.shuffle(cols)
    return cols[:n] if n <= len(cols) else (cols * ((n + len(cols) - 1) // len(cols)))[:n]


def onehot_x(T, H, cols, vals, x_dtype):
    x = np.zeros((T, H), dtype=np.float64)
    for t in range(T):
        x[t, cols[t]] = vals[t]
    return synth.f64_to_bf16_bits(x) if x_dtype == "bf16" else x.astype(np.float32)


def fc1_onehot(v, dev, T, cols, vals, x_dtype="bf16", step=None):
    """route + FC1 on one-hot tokens; every h element against silu(v W_g[:, j]) * v W_u[:, j]."""
    H, k = dev.hidden, dev.top_k
    st = step or Step(dev, T)
    xt = x_tensor(onehot_x(T, H, cols, vals, x_dtype), x_dtype)
    st.route(xt)
    st.fc1(xt)
    torch.cuda.synchronize()
    status, info = st.check()
    assert status == _lib.OK, (status, info)
    ids = st.ids[:T].cpu().numpy()
    h = st.h[:T * k].cpu().numpy().astype(np.float64).reshape(T, k, -1)
    dec = Decoded(v)
    worst = 0.0
    for t in range(T):
        for i in range(k):
            Wg, Wu, _ = dec(int(ids[t, i]))
            g = vals[t] * Wg[:, cols[t]]
            u = vals[t] * Wu[:, cols[t]]
            ref = oracle.silu(g) * u
            err = np.abs(h[t, i] - ref)
            bad = err > H_TOL * np.abs(ref) + 2.0 ** -126
            assert not bad.any(), (f"token {t} (column {cols[t]}), expert {ids[t, i]}: rows "
                                   f"{np.nonzero(bad)[0][:8].tolist()} off, e.g. {h[t, i][bad][:3]} vs {ref[bad][:3]}")
            worst = max(worst, float((err / np.maximum(np.abs(ref), 1e-300)).max()))
    return worst, ids


def fc2_onehot(v, dev, T, cols, vals, seed=0, step=None):
    """route (any tokens) + FC2 on a one-hot h; y against sum_i w_i v_i W_d,i[:, j_i]."""
    H, I, k = dev.hidden, dev.inter, dev.top_k
    st = step or Step(dev, T)
    x = synth.f64_to_bf16_bits(np.random.default_rng(seed).standard_normal((T, H)))
    xt = x_tensor(x, "bf16")
    st.route(xt)
    hz = torch.zeros((T * k, I), dtype=torch.float32)
    for p in range(T * k):
        hz[p, cols[p]] = float(vals[p])
    st.h[:T * k].copy_(hz)
    st.fc2(T)
    torch.cuda.synchronize()
    status, info = st.check()
    assert status == _lib.OK, (status, info)
    ids = st.ids[:T].cpu().numpy()
    w = st.w[:T].cpu().numpy().astype(np.float64)
    y = st.y[:T].cpu().numpy().astype(np.float64)
    dec = Decoded(v)
    worst = 0.0
    for t in range(T):
        terms = np.stack([w[t, i] * vals[t * k + i] * dec(int(ids[t, i]))[2][:, cols[t * k + i]] for i in range(k)])
        ref = terms.sum(axis=0)
        mag = np.abs(terms).sum(axis=0)
        err = np.abs(y[t] - ref)
        bad = err > Y_TOL * mag + 2.0 ** -126
        assert not bad.any(), (f"token {t}: rows {np.nonzero(bad)[0][:8].tolist()} off, "
                               f"e.g. {y[t][bad][:3]} vs {ref[bad][:3]}")
        worst = max(worst, float((err / np.maximum(mag, 1e-300)).max()))
    return worst, ids


POW2 = [1.0, -1.0, 2.0, -0.5, 4.0, -2.0, 0.25, 1.0]


@pytest.mark.parametrize("name", list(LAYERS))
@pytest.mark.parametrize("mixed", [False, True])
def test_fc1_onehot_every_kernel(name, mixed):
    """T = 1 (one-token kernels), then T = 12 and 40 tokens (token-group kernels), each
    token hot at its own column."""
    v, dev = make_layer(name, mixed=mixed)
    H = dev.hidden
    for T, seed in ((1, 1), (1, 2), (1, 3), (12, 4), (40, 5)):
        cols = spread_columns(H, T, seed) if T > 1 else [[0, H // 2 + 5, H - 1][seed - 1]]
        vals = [POW2[(t + seed) % len(POW2)] for t in range(T)]
        say(f"fc1 one-hot {name} mixed={mixed} T={T}")
        worst, _ = fc1_onehot(v, dev, T, cols, vals)
        say(f"  worst relative h error {worst:.2e}")


@pytest.mark.parametrize("name", list(LAYERS))
@pytest.mark.parametrize("mixed", [False, True])
def test_fc2_onehot_every_kernel(name, mixed):
    v, dev = make_layer(name, mixed=mixed)
    I, k = dev.inter, dev.top_k
    for T, seed in ((1, 11), (1, 12), (12, 13), (40, 14)):
        cols = spread_columns(I, T * k, seed)
        vals = [POW2[(p + seed) % len(POW2)] for p in range(T * k)]
        say(f"fc2 one-hot {name} mixed={mixed} T={T}")
        worst, _ = fc2_onehot(v, dev, T, cols, vals, seed=seed)
        say(f"  worst error / sum of term magnitudes {worst:.2e}")


@pytest.mark.parametrize("name", ["h2048_i1024", "h1024_i2048", "h7168_i2048", "h2048_i1024_k12"])
@pytest.mark.parametrize("mixed", [False, True])
def test_forward_one_token_onehot(name, mixed):
    """moe_vq_forward at one token: every h element against the oracle's decode, and y
    against the three-call step bit for bit."""
    v, dev = make_layer(name, mixed=mixed)
    H, k = dev.hidden, dev.top_k
    dec = Decoded(v)
    for j, val in ((0, 1.0), (H // 2 + 5, -2.0), (H - 1, 0.5)):
        xt = x_tensor(onehot_x(1, H, [j], [val], "bf16"), "bf16")
        st = Step(dev, 1)
        y = st.step(xt).clone()
        torch.cuda.synchronize()
        assert st.check()[0] == _lib.OK
        ids = st.ids[:1].cpu().numpy()
        h = st.h[:k].cpu().numpy().astype(np.float64)
        for i in range(k):
            Wg, Wu, _ = dec(int(ids[0, i]))
            ref = oracle.silu(val * Wg[:, j]) * (val * Wu[:, j])
            bad = np.abs(h[i] - ref) > H_TOL * np.abs(ref) + 2.0 ** -126
            assert not bad.any(), (name, j, i, np.nonzero(bad)[0][:8].tolist())
        g = run(dev, onehot_x(1, H, [j], [val], "bf16"), "bf16")
        assert np.array_equal(g["ids"], ids) and np.array_equal(g["y"], y.cpu().numpy().astype(np.float64))


def test_forward_one_token_absent_experts():
    """moe_vq_forward at one token reports the lowest absent selected expert and leaves it
    out of y."""
    v0, dev0 = make_layer("h2048_i1024")
    x = synth.f64_to_bf16_bits(np.random.default_rng(77).standard_normal((1, 2048)))
    st0 = Step(dev0, 1)
    st0.step(x_tensor(x, "bf16"))
    ids = st0.ids[0].cpu().numpy()
    gone = sorted(int(e) for e in ids[1:3])
    fm = [synth.FMT_VQ2] * 16
    for e in gone:
        fm[e] = synth.FMT_ABSENT
    v, dev = tiny_variant(v0, formats=fm)
    st = Step(dev, 1)
    y = st.step(x_tensor(x, "bf16")).cpu().numpy().astype(np.float64)
    status, info = st.check()
    assert status == _lib.ENOTRESIDENT and info == gone[0]
    r = oracle.forward(v0, oracle.x_value(x, "bf16"), 4, forced_selection=st.ids[:1].cpu().numpy())
    keep = ~np.isin(st.ids[:1].cpu().numpy(), gone)[:, :, None]
    y_ref = (r["w"][:, :, None] * r["o"] * keep).sum(axis=1)
    assert (np.abs(y - y_ref).max() / np.abs(y_ref).max()) <= 1e-2


def test_fc1_onehot_fp32_activations():
    v, dev = make_layer("h2048_i1024")
    for T in (1, 12):
        cols = spread_columns(dev.hidden, T, 21)
        fc1_onehot(v, dev, T, cols, [POW2[t % 8] for t in range(T)], x_dtype="f32")


def _up_only_row(n0):
    """Zero every row of every expert's up matrix except row n0 (VQ2: zero scales; MXFP4:
    zero E2M1 codes), so that h is one-hot at n0."""
    def mutate(experts):
        for e, ex in experts.items():
            if int(ex["format"]) == synth.FMT_VQ2:
                s = np.zeros_like(ex["scales_u"])
                s[n0] = ex["scales_u"][n0]
                ex["scales_u"] = s
            else:
                q = np.zeros_like(ex["nib_u"])
                q[n0] = ex["nib_u"][n0]
                ex["nib_u"] = q
    return mutate


@pytest.mark.parametrize("name,n0", [("h2048_i1024", 0), ("h2048_i1024", 517), ("h1024_i2048", 2047),
                                     ("h384_i640", 300)])
@pytest.mark.parametrize("mixed", [False, True])
def test_prefill_onehot_isolates_weights(name, n0, mixed):
    v, dev = make_layer(name, mixed=mixed, mutate=_up_only_row(n0))
    H, k = dev.hidden, dev.top_k
    T = 70
    cols = spread_columns(H, T, 31 + n0)
    vals = [POW2[t % 8] for t in range(T)]
    x = onehot_x(T, H, cols, vals, "bf16")
    say(f"prefill one-hot {name} n0={n0} mixed={mixed}")
    g = run_prefill(dev, x, "bf16")
    assert g["status"] == _lib.OK
    dec = Decoded(v)
    for t in range(T):
        terms = []
        for i in range(k):
            Wg, Wu, Wd = dec(int(g["ids"][t, i]))
            hn0 = oracle.silu(vals[t] * Wg[n0, cols[t]]) * (vals[t] * Wu[n0, cols[t]])
            terms.append(g["w"][t, i] * hn0 * Wd[:, n0])
        terms = np.stack(terms)
        ref, mag = terms.sum(axis=0), np.abs(terms).sum(axis=0)
        bad = np.abs(g["y"][t] - ref) > 5e-3 * mag + 2.0 ** -126
        assert not bad.any(), (t, cols[t], np.nonzero(bad)[0][:8].tolist())


# ---------------------------------------------------------------------------------
# MXFP4 with E8M0 exponents far from 127: the matrix-core paths scale each block by
# 2^(e - e_max) before the fp16 convert, so no exponent overflows or underflows there
# ---------------------------------------------------------------------------------

def _shift_e8m0(kind):
    def mutate(experts):
        for e, ex in experts.items():
            if int(ex["format"]) != synth.FMT_MXFP4:
                continue
            rng = np.random.default_rng(900 + e)
            for key in ("e8m0_g", "e8m0_u", "e8m0_d"):
                a = ex[key].astype(np.int64)
                if kind == "high":
                    a = a + 22 + (e % 2) * 3            # 140 .. 145
                elif kind == "low":
                    a = a - 14 - (e % 2) * 4             # 100 .. 106
                else:                                    # mixed blocks within one group
                    a = rng.choice(np.array([100, 104, 118, 140, 145]), size=a.shape)
                ex[key] = a.astype(np.uint8)
    return mutate


@pytest.mark.parametrize("kind", ["high", "low", "mixed"])
def test_mxfp4_extreme_exponents(kind):
    cfg = synth.Config("mx_range", 4, 2048, 1024, 8, 2, "bf16", "normal", seed=6060)
    syn = synth.SynthLayer(cfg, cache=False)
    v, dev = tiny_variant(syn, formats=[synth.FMT_MXFP4] * 8, mutate=_shift_e8m0(kind))
    for T in (1, 9, 40):
        x = syn.x(n=T, stream=700 + T)
        say(f"mxfp4 exponents {kind}, decode path T={T}")
        gd = run(dev, x, "bf16")
        assert gd["status"] == _lib.OK
        compare(v, x, "bf16", gd, cfg.top_k)
        say(f"mxfp4 exponents {kind}, prefill T={T}")
        gp = run_prefill(dev, x, "bf16")
        assert gp["status"] == _lib.OK
        compare(v, x, "bf16", gp, cfg.top_k, check_h=False)
    # one-hot x: every h element exact to the SiLU rounding, also far from 2^0
    if kind != "mixed":
        cols = spread_columns(2048, 12, 77)
        fc1_onehot(v, dev, 12, cols, [1.0] * 12)
        fc1_onehot(v, dev, 1, [1000], [1.0])


# ---------------------------------------------------------------------------------
# A workspace routed for other shapes or other activations: the compute call is refused
# on the device and moe_vq_check reports MOE_VQ_EINVAL
# ---------------------------------------------------------------------------------

def _raw_fc1(st, xt, T):
    return _lib.raw().moe_vq_fc1_silu(st.layer.c, xt.data_ptr(), _lib.BF16 if xt.dtype == torch.bfloat16 else _lib.F32,
                                      T, st.ws.data_ptr(), st.ws_bytes, st.h.data_ptr(), st.stream())


def _raw_fc2(st, T):
    return _lib.raw().moe_vq_fc2_combine(st.layer.c, st.h.data_ptr(), T, st.ws.data_ptr(), st.ws_bytes,
                                         st.y.data_ptr(), st.stream())


def _raw_prefill(st, xt, T):
    return _lib.raw().moe_vq_prefill_gemm(st.layer.c, xt.data_ptr(), _lib.BF16 if xt.dtype == torch.bfloat16 else _lib.F32,
                                          T, st.ws.data_ptr(), st.ws_bytes, st.y.data_ptr(), st.stream())


@pytest.mark.parametrize("name,T", [("h2048_i1024", 1), ("h2048_i1024", 4), ("h256_i128", 4), ("h7168_i2048", 1)])
def test_workspace_mismatch_is_reported(name, T):
    v, dev = make_layer(name)
    H = dev.hidden
    st = Step(dev, T + 1)
    x = synth.f64_to_bf16_bits(np.random.default_rng(5).standard_normal((T + 1, H)))
    xa = x_tensor(x[:T], "bf16")
    xb = x_tensor(x[:T + 1], "bf16")
    # routed for T tokens, called for T + 1
    st.route(xa)
    assert st.check()[0] == _lib.OK
    assert _raw_fc1(st, xb, T + 1) == _lib.OK  # (accepted on the host: the workspace is large enough)
    assert st.check()[0] == _lib.EINVAL
    st.route(xa)
    assert _raw_fc2(st, T + 1) == _lib.OK
    assert st.check()[0] == _lib.EINVAL
    st.route(xa)
    assert _raw_prefill(st, xb, T + 1) == _lib.OK
    assert st.check()[0] == _lib.EINVAL
    # same shapes, other activations (a copy of the same values at another address)
    st.route(xa)
    assert _raw_fc1(st, xa.clone(), T) == _lib.OK
    assert st.check()[0] == _lib.EINVAL
    st.route(xa)
    assert _raw_prefill(st, xa.clone(), T) == _lib.OK
    assert st.check()[0] == _lib.EINVAL
    # routed again properly: the step runs and checks OK
    g = run(dev, x[:T], "bf16", step=st)
    assert g["status"] == _lib.OK
    compare(v, x[:T], "bf16", g, dev.top_k)
