"""Host-RAM expert tier on the GPU: a layer with every expert in a pinned host pool and
only some device slots gives, step after step, the same bits as the layer with every
expert resident (the kernels read the same bytes), while experts are copied in and
evicted, and every tiered step matches the fp64 oracle under the parity rules; a step
selecting more experts than the tier has slots is refused."""
import numpy as np
import pytest
import torch

import synth
from bit_vector_quantised_amd import _lib
from bit_vector_quantised_amd.layer import DeviceLayer, Step, TieredLayer, tiered_forward

from gpu_util import compare, say, x_tensor

pytestmark = pytest.mark.gpu

MINI = synth.Config("mini", 6, 2048, 1024, 16, 4, "bf16", "normal", seed=4242)


@pytest.fixture(scope="module")
def mini_syn():
    return synth.SynthLayer(MINI)


@pytest.mark.parametrize("mixed", [False, True])
def test_tier_steps_match_all_resident_bits(mini_syn, mixed):
    syn = mini_syn
    fm = [(_lib.FMT_MXFP4 if e % 3 == 0 else _lib.FMT_VQ2) for e in range(MINI.n_experts)] if mixed else None
    full = DeviceLayer.from_synth(syn, formats=fm)
    tiered = TieredLayer.from_synth(syn, n_dev_slots=8, formats=fm)
    st_full, st_tier = Step(full, 2), Step(tiered, 2)

    class View:  # the layer as the oracle reads it: each expert in its slot's format
        pass
    view = View()
    view.cfg, view.codebook, view.router_w = syn.cfg, syn.codebook, syn.router_w
    fmts = fm if fm is not None else list(syn.formats)
    view.expert = lambda e: syn.expert_as(e, fmts[e])
    copied, hits = 0, 0
    # each input twice in a row: the repeat finds its experts resident
    for i, T in enumerate([1, 1, 2, 2, 1, 1, 1, 1, 2, 2, 1, 1]):
        say(f"tier step {i} T={T} mixed={mixed}")
        x_np = syn.x(n=T, stream=300 + i // 2)
        x = x_tensor(x_np, "bf16")
        y_ref = st_full.forward(x).clone()
        y, n = tiered_forward(st_tier, tiered, x)
        torch.cuda.synchronize()
        assert st_full.check()[0] == _lib.OK
        assert st_tier.check()[0] == _lib.OK, "an expert the step selected is still absent"
        assert torch.equal(y, y_ref), f"step {i}: tiered output differs from the all-resident one"
        assert torch.equal(st_tier.ids[:T], st_full.ids[:T])
        g = {"ids": st_tier.ids[:T].cpu().numpy().astype(np.int64),
             "w": st_tier.w[:T].cpu().numpy().astype(np.float64),
             "h": st_tier.h[:T * MINI.top_k].cpu().numpy().astype(np.float64).reshape(T, MINI.top_k, -1),
             "y": y.cpu().numpy().astype(np.float64)}
        compare(view, x_np, "bf16", g, MINI.top_k)
        copied += n
        if i % 2 == 1:
            assert n == 0, "a repeated step copied experts"
            hits += 1
    held = [e for e in tiered.tier.held() if e >= 0]
    assert len(held) == len(set(held)) <= 8
    assert copied > 8, "the sequence should have evicted experts"


def test_tier_refuses_a_step_wider_than_its_slots(mini_syn):
    syn = mini_syn
    tiered = TieredLayer.from_synth(syn, n_dev_slots=3)  # one token selects top_k = 4 experts
    st = Step(tiered, 1)
    st.route(x_tensor(syn.x(n=1, stream=400), "bf16"))
    with pytest.raises(_lib.MoeVqError) as ei:
        _lib.tier_resolve(tiered.c, tiered.tier, tiered.pool.data_ptr(), tiered.slots.data_ptr(), 1,
                          st.ws.data_ptr(), st.stream())
    assert ei.value.status == _lib.ENOSPACE
    assert tiered.tier.held() == [-1, -1, -1]


@pytest.mark.parametrize("T", [1, 5, 33])
def test_step_info_reads_the_selection(mini_syn, T):
    """moe_vq_step_info (and the tier's read of a step, which shares it) returns the
    step's status, its distinct experts in ascending order and its pair count."""
    say(f"step_info T={T}")
    dev = DeviceLayer.from_synth(mini_syn)
    st = Step(dev, T)
    x = x_tensor(mini_syn.x(n=T, stream=900 + T), "bf16")
    st.route(x)
    info = _lib.step_info(dev.c, T, st.ws.data_ptr(), st.stream())
    ids = st.ids[:T].cpu().numpy()
    want = sorted(set(int(e) for e in ids.ravel()))
    assert info["status"] == _lib.OK and info["info"] == -1
    assert info["experts"] == want and info["n_active"] == len(want)
    assert info["n_pairs"] == T * MINI.top_k
