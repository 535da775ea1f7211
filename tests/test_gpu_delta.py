"""FP4 delta cache with a confidence gate on the GPU: a routed pair whose weight reaches
the gate, and whose expert has an FP4 copy, is computed from the copy.  Checked against
the fp64 oracle under the parity rules, on every decode kernel and on prefill; with the
gate at 0 and a copy of every expert the step is bit-identical to the layer stored in
FP4, and with the gate above 1 to the layer without the cache."""
import numpy as np
import pytest
import torch

import synth
from bit_vector_quantised_amd import _lib
from bit_vector_quantised_amd.layer import DeviceLayer, Step

from gpu_util import compare, run, run_prefill, say

pytestmark = pytest.mark.gpu

MINI = synth.Config("mini", 6, 2048, 1024, 16, 4, "bf16", "normal", seed=4242)
WIDE = synth.Config("wide", 6, 7168, 2048, 16, 4, "bf16", "normal", seed=777)
GAP = 1e-4  # no routing weight may lie this close to the gate (both sides then decide alike)


@pytest.fixture(scope="module")
def mini_syn():
    return synth.SynthLayer(MINI)


def copies_of(syn, experts):
    have = set(int(e) for e in experts)
    return lambda e: syn.expert_as(e, synth.FMT_MXFP4) if e in have else None


def gate_between(w, q):
    """A gate at quantile q of the step's routing weights, in the middle of the gap around
    it; the gap must leave every weight at least GAP away."""
    s = np.unique(np.sort(np.asarray(w, dtype=np.float64).reshape(-1)))
    i = int(np.clip(round(q * (len(s) - 1)), 0, len(s) - 2))
    while i < len(s) - 2 and s[i + 1] - s[i] < 2 * GAP:
        i += 1
    tau = 0.5 * (s[i] + s[i + 1])
    assert np.abs(s - tau).min() >= GAP, "no gap wide enough in the routing weights"
    return float(tau)


def listed_copies(dev, st, T):
    """The FP4 copies the step listed (experts E + e, returned as e)."""
    inf = _lib.step_info(dev.c, T, st.ws.data_ptr(), st.stream())
    return sorted(e - dev.n_experts for e in inf["experts"] if e >= dev.n_experts)


def check_step(syn, dev, cp, tau, x_np, T, tokens=None):
    g = run(dev, x_np, "bf16")
    assert g["status"] == _lib.OK, (g["status"], g["info"])
    r = compare(syn, x_np, "bf16", g, syn.cfg.top_k, tokens=tokens, fp4_copy=cp, gate_tau=tau)["ref"]
    assert np.abs(g["w"] - tau).min() >= GAP / 2
    if tokens is None:  # the copies the GPU listed are exactly those the oracle used
        used = sorted(set(int(e) for e in r["ids"][r["copy"]]))
        assert listed_copies(dev, g["step"], T) == used
    return g, r


@pytest.mark.parametrize("T", [1, 3, 24, 40])
def test_gated_steps_match_oracle(mini_syn, T):
    """Copies for the even experts, the gate inside the step's weight range: both gated
    and ungated pairs occur, on the one-token kernels (T = 1), the matrix-core decode
    kernel (T > 1) and its ragged groups."""
    syn = mini_syn
    say(f"delta mini T={T}")
    x_np = syn.x(n=T, stream=500 + T)
    plain = run(DeviceLayer.from_synth(syn), x_np, "bf16")
    tau = gate_between(plain["w"], 0.0 if T == 1 else 0.7)
    cp = copies_of(syn, range(0, MINI.n_experts, 2))
    dev = DeviceLayer.from_synth(syn, fp4_copies=range(0, MINI.n_experts, 2), gate_tau=tau)
    g, r = check_step(syn, dev, cp, tau, x_np, T)
    assert r["copy"].any()
    if T > 1:
        assert (~r["copy"]).any()


@pytest.mark.parametrize("T", [1, 5, 32])
def test_gate_zero_with_every_copy_is_the_fp4_layer_bitwise(mini_syn, T):
    """Gate 0, a copy of every expert: every pair reads its copy, so h and y are the bits
    of the same step on the layer whose experts are all stored in FP4."""
    syn = mini_syn
    say(f"delta all-copies T={T}")
    E = MINI.n_experts
    x_np = syn.x(n=T, stream=600 + T)
    dev = DeviceLayer.from_synth(syn, fp4_copies=range(E), gate_tau=0.0)
    fp4 = DeviceLayer.from_synth(syn, formats=[synth.FMT_MXFP4] * E)
    g, g4 = run(dev, x_np, "bf16"), run(fp4, x_np, "bf16")
    assert g["status"] == _lib.OK and g4["status"] == _lib.OK
    assert np.array_equal(g["ids"], g4["ids"])
    assert np.array_equal(g["h"], g4["h"]) and np.array_equal(g["y"], g4["y"])
    assert listed_copies(dev, g["step"], T) == sorted(set(g["ids"].reshape(-1).tolist()))


@pytest.mark.parametrize("T", [1, 7])
def test_gate_above_one_is_the_plain_layer_bitwise(mini_syn, T):
    syn = mini_syn
    say(f"delta gate>1 T={T}")
    x_np = syn.x(n=T, stream=700 + T)
    dev = DeviceLayer.from_synth(syn, fp4_copies=range(MINI.n_experts), gate_tau=1.5)
    g, g0 = run(dev, x_np, "bf16"), run(DeviceLayer.from_synth(syn), x_np, "bf16")
    assert g["status"] == _lib.OK
    assert np.array_equal(g["h"], g0["h"]) and np.array_equal(g["y"], g0["y"])
    assert listed_copies(dev, g["step"], T) == []


def test_bad_copy_slot_is_reported_as_its_listed_expert(mini_syn):
    """A copy whose slot lies outside the pool is reported (MOE_VQ_ENOTRESIDENT) under its
    listed id E + e and left out of y; an absent copy is no error (the pair keeps its
    2-bit expert)."""
    syn = mini_syn
    say("delta bad copy slot")
    E = MINI.n_experts
    x_np = syn.x(n=1, stream=801)
    dev = DeviceLayer.from_synth(syn, fp4_copies=range(E), gate_tau=0.0)
    g = run(dev, x_np, "bf16")
    e0 = int(g["ids"][0, 0])
    tab = dev.delta_slots.cpu().numpy().view(
        [("byte_offset", "<u8"), ("format", "<u4"), ("reserved", "<u4")]).copy()
    tab["byte_offset"][e0] = dev.pool_bytes + 256
    dev.delta_slots.copy_(torch.from_numpy(tab.view(np.uint8)))
    g = run(dev, x_np, "bf16", step=g["step"])
    assert g["status"] == _lib.ENOTRESIDENT and g["info"] == E + e0
    tab["format"][:] = _lib.FMT_ABSENT
    dev.delta_slots.copy_(torch.from_numpy(tab.view(np.uint8)))
    g = run(dev, x_np, "bf16", step=g["step"])
    g0 = run(DeviceLayer.from_synth(syn), x_np, "bf16")
    assert g["status"] == _lib.OK and np.array_equal(g["y"], g0["y"])


@pytest.mark.parametrize("T", [1, 40])
def test_gated_steps_match_oracle_at_k_7168(T):
    """H = 7168: the one-token stream kernel's and the matrix-core kernel's FC1 at K =
    7168 with gated pairs."""
    syn = synth.SynthLayer(WIDE)
    say(f"delta wide T={T}")
    x_np = syn.x(n=T, stream=900 + T)
    plain = run(DeviceLayer.from_synth(syn), x_np, "bf16")
    tau = gate_between(plain["w"], 0.0 if T == 1 else 0.6)
    have = range(1, WIDE.n_experts, 2)
    dev = DeviceLayer.from_synth(syn, fp4_copies=have, gate_tau=tau)
    g, r = check_step(syn, dev, copies_of(syn, have), tau, x_np, T, tokens=None if T == 1 else [0, 7, 39])


def test_prefill_with_gated_pairs(mini_syn):
    """The prefill GEMMs read the copies through the same worklist: sampled tokens match
    the oracle, and with gate 0 and every copy y is the all-FP4 layer's prefill, bit for
    bit."""
    syn = mini_syn
    T = 300
    say(f"delta prefill T={T}")
    E = MINI.n_experts
    x_np = syn.x(n=T, stream=1000)
    plain = run_prefill(DeviceLayer.from_synth(syn), x_np, "bf16")
    tau = gate_between(plain["w"], 0.8)
    have = range(0, E, 2)
    dev = DeviceLayer.from_synth(syn, fp4_copies=have, gate_tau=tau)
    g = run_prefill(dev, x_np, "bf16")
    assert g["status"] == _lib.OK
    r = compare(syn, x_np, "bf16", g, MINI.top_k, tokens=list(range(0, T, 10)), check_h=False,
                fp4_copy=copies_of(syn, have), gate_tau=tau)["ref"]
    assert r["copy"].any() and (~r["copy"]).any()
    dev0 = DeviceLayer.from_synth(syn, fp4_copies=range(E), gate_tau=0.0)
    fp4 = DeviceLayer.from_synth(syn, formats=[synth.FMT_MXFP4] * E)
    a, b = run_prefill(dev0, x_np, "bf16"), run_prefill(fp4, x_np, "bf16")
    assert np.array_equal(a["y"], b["y"])
