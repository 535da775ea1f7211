"""The measurement hook moe_vq_time_next_kernel: an FC kernel launched through it gives
the same bits as a plain launch, its events bracket a positive run time, and the hook is
used by exactly one launch."""
import pytest
import torch

import synth
from bit_vector_quantised_amd import _lib
from bit_vector_quantised_amd.layer import DeviceLayer, Step

from gpu_util import say, x_tensor

pytestmark = pytest.mark.gpu

MINI = synth.Config("mini", 6, 2048, 1024, 16, 4, "bf16", "normal", seed=4242)


@pytest.mark.parametrize("T", [1, 24])
def test_timed_launch_matches_plain_launch(T):
    say(f"timing hook T={T}")
    syn = synth.SynthLayer(MINI)
    dev = DeviceLayer.from_synth(syn)
    st = Step(dev, T)
    x = x_tensor(syn.x(n=T, stream=77), "bf16")
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in ev:
        e.record(stream)
    torch.cuda.synchronize()

    st.route(x)
    st.fc1(x)
    st.fc2(T)
    torch.cuda.synchronize()
    h_ref, y_ref = st.h[:T * MINI.top_k].clone(), st.y[:T].clone()

    st.route(x)
    _lib.time_next_kernel(ev[0].cuda_event, ev[1].cuda_event)
    st.fc1(x)
    _lib.time_next_kernel(ev[2].cuda_event, ev[3].cuda_event)
    st.fc2(T)
    torch.cuda.synchronize()
    assert st.check()[0] == _lib.OK
    assert torch.equal(st.h[:T * MINI.top_k], h_ref)
    assert torch.equal(st.y[:T], y_ref)
    fc1_ms, fc2_ms = ev[0].elapsed_time(ev[1]), ev[2].elapsed_time(ev[3])
    assert 0 < fc1_ms < 50 and 0 < fc2_ms < 50, (fc1_ms, fc2_ms)

    # used once: the next launches do not touch the events again
    st.route(x)
    st.fc1(x)
    st.fc2(T)
    torch.cuda.synchronize()
    assert ev[0].elapsed_time(ev[1]) == fc1_ms and ev[2].elapsed_time(ev[3]) == fc2_ms
    _lib.time_next_kernel(0, 0)


def test_read_probe_runs_and_is_timed_by_the_hook():
    """The streaming read probe reads a buffer (its sink stays untouched for zero data) and
    its launch records the hook's events; 64 MiB take well under a millisecond."""
    say("read probe")
    buf = torch.zeros(16 << 20, dtype=torch.int32, device="cuda")
    sink = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    b.record(stream)
    torch.cuda.synchronize()
    _lib.time_next_kernel(a.cuda_event, b.cuda_event)
    _lib.read_probe(buf.data_ptr(), buf.numel() * 4, sink.data_ptr(), stream.cuda_stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b)
    assert 0 < ms < 1.0, ms
    assert int(sink.item()) == 7
    say("read probe GB/s", buf.numel() * 4 / (ms * 1e-3) / 1e9)
