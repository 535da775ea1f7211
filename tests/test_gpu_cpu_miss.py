"""The CPU miss path on the GPU: a tiered layer whose device slots hold some of the
experts; each step's other selected experts are computed on the host cores from the host
pool while the GPU runs the resident ones, and y is their sum.  Every step is compared with
the fp64 oracle (the parity rules) and with the layer whose experts are all resident."""
import numpy as np
import pytest
import torch

import synth
from bit_vector_quantised_amd import _lib
from bit_vector_quantised_amd.layer import DeviceLayer, Step, TieredLayer, cpu_miss_forward, tiered_forward

from gpu_util import compare, say, x_tensor

pytestmark = pytest.mark.gpu

MINI = synth.Config("mini", 6, 2048, 1024, 16, 4, "bf16", "normal", seed=4242)


@pytest.mark.parametrize("mixed", [False, True])
def test_cpu_miss_steps_match_oracle_and_resident(mixed):
    syn = synth.SynthLayer(MINI)
    fm = [(_lib.FMT_MXFP4 if e % 3 == 0 else _lib.FMT_VQ2) for e in range(MINI.n_experts)] if mixed else None
    fmts = fm if fm is not None else list(syn.formats)
    full = DeviceLayer.from_synth(syn, formats=fm)
    tiered = TieredLayer.from_synth(syn, n_dev_slots=8, formats=fm)
    st_full, st_tier = Step(full, 6), Step(tiered, 6)

    class View:
        pass
    view = View()
    view.cfg, view.codebook, view.router_w = syn.cfg, syn.codebook, syn.router_w
    view.expert = lambda e: syn.expert_as(e, fmts[e])
    # fill some device slots through the copying tier first
    for i in range(3):
        tiered_forward(st_tier, tiered, x_tensor(syn.x(n=2, stream=600 + i), "bf16"))
    missed_total = 0
    for i, T in enumerate([1, 2, 5, 6, 1]):
        say(f"cpu miss step {i} T={T} mixed={mixed}")
        x_np = syn.x(n=T, stream=700 + i)
        x = x_tensor(x_np, "bf16")
        y_ref = st_full.forward(x).clone()
        y, miss = cpu_miss_forward(st_tier, tiered, x, n_threads=8)
        torch.cuda.synchronize()
        status, info = st_tier.check()
        if miss:
            assert status == _lib.ENOTRESIDENT and info == miss[0]
        else:
            assert status == _lib.OK
        missed_total += len(miss)
        assert torch.equal(st_tier.ids[:T], st_full.ids[:T])
        g = {"ids": st_tier.ids[:T].cpu().numpy().astype(np.int64),
             "w": st_tier.w[:T].cpu().numpy().astype(np.float64),
             "y": y.cpu().numpy().astype(np.float64)}
        compare(view, x_np, "bf16", g, MINI.top_k, check_h=False)
        d = (y - y_ref).abs().max(dim=1).values / y_ref.abs().max(dim=1).values
        assert float(d.max()) <= 1e-2
    assert missed_total > 0, "the sequence should have computed experts on the host"
