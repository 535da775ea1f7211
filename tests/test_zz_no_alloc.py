"""The no-allocation entry point moe_vq_forward_static (workspace in the library's static
device array) against moe_vq_forward (caller workspace), through the C ABI: two calls in a
row, the second with fewer tokens, bit for bit equal outputs and status; a step whose
workspace exceeds the array is refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from bit_vector_quantised_amd import _lib
from bit_vector_quantised_amd.layer import DeviceLayer, Step

from gpu_util import say, x_tensor

pytestmark = pytest.mark.gpu

LAYER = synth.Config("noalloc", 12, 2048, 1024, 16, 4, "bf16", "normal", seed=8181)


def _static_call(dev, xt, T):
    k, I, H = dev.top_k, dev.inter, dev.hidden
    ids = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    w = torch.full((T, k), -1.0, dtype=torch.float32, device="cuda")
    h = torch.full((T * k, I), -1.0, dtype=torch.float32, device="cuda")
    y = torch.full((T, H), -1.0, dtype=torch.float32, device="cuda")
    status = torch.full((2,), -7, dtype=torch.int32, device="cuda")
    rc = _lib.raw().moe_vq_forward_static(ctypes.byref(dev.c), xt.data_ptr(), _lib.BF16, T, ids.data_ptr(),
                                          w.data_ptr(), h.data_ptr(), y.data_ptr(), status.data_ptr(),
                                          torch.cuda.current_stream().cuda_stream)
    assert rc == _lib.OK, rc
    torch.cuda.synchronize()
    return ids, w, h, y, status.cpu().tolist()


def test_forward_static_matches_forward_twice_second_smaller():
    syn = synth.SynthLayer(LAYER)
    dev = DeviceLayer.from_synth(syn)
    for T, stream in ((12, 1), (3, 2)):
        say(f"no-alloc entry point, T={T}")
        xt = x_tensor(syn.x(n=T, stream=stream), "bf16")
        ref = Step(dev, T)
        y_ref = ref.step(xt)
        st_ref = ref.check()
        ids, w, h, y, status = _static_call(dev, xt, T)
        assert status == [st_ref[0], st_ref[1]] == [_lib.OK, -1]
        assert torch.equal(ids, ref.ids[:T])
        assert torch.equal(w, ref.w[:T])
        assert torch.equal(h, ref.h[:T * dev.top_k])
        assert torch.equal(y, y_ref)


def test_forward_static_reports_absent_expert_and_refuses_oversize():
    syn = synth.SynthLayer(LAYER)
    fm = list(syn.formats)
    xt = x_tensor(syn.x(n=4, stream=3), "bf16")
    dev0 = DeviceLayer.from_synth(syn)
    ids0, _, _, _, _ = _static_call(dev0, xt, 4)
    gone = int(ids0[0, 0].item())
    fm[gone] = synth.FMT_ABSENT
    dev = DeviceLayer.from_synth(syn, formats=fm)
    _, _, _, _, status = _static_call(dev, xt, 4)
    assert status[0] == _lib.ENOTRESIDENT
    # the full-size shape at 64 tokens needs 18.3 MiB of workspace: more than the array holds
    big = _lib.Layer(7168, 2048, 256, 8, dev.c.router_w, dev.c.codebook, dev.c.pool, dev.c.pool_bytes, dev.c.slots)
    assert _lib.workspace_bytes(big, 64) > 16 << 20
    assert _lib.workspace_bytes(big, 32) <= 16 << 20
    rc = _lib.raw().moe_vq_forward_static(ctypes.byref(big), xt.data_ptr(), _lib.BF16, 64, 0x1000, 0x1000,
                                          0x1000, 0x1000, None, None)
    assert rc == _lib.ENOSPACE
