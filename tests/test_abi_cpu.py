"""The C-ABI library on a machine without a GPU: it loads, exports every declared
symbol, computes sizes and layouts, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_vq.h")

mvq = pytest.importorskip("bit_vector_quantised_amd")
from bit_vector_quantised_amd import _lib  # noqa: E402
from bit_vector_quantised_amd.layer import pack_slot  # noqa: E402


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_vq_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert "moe_vq_route_topk" in names and "moe_vq_fc1_silu" in names and len(names) >= 10
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.EXPORTS)


def test_only_the_c_api_is_exported():
    """Internal (C++) functions stay hidden: a second copy of the library in the same
    process cannot take them over."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True, check=True).stdout
    funcs = sorted({ln.split()[-1] for ln in out.splitlines() if len(ln.split()) == 3 and ln.split()[1] in "TW"})
    assert funcs and all(f.startswith("moe_vq_") for f in funcs), [f for f in funcs if not f.startswith("moe_vq_")][:10]
    assert set(funcs) == set(declared_functions())


def test_expert_bytes():
    assert _lib.expert_bytes(_lib.FMT_VQ2, 7168, 2048) == 11_698_176
    assert _lib.expert_bytes(_lib.FMT_MXFP4, 7168, 2048) == 23_396_352
    assert _lib.expert_bytes(_lib.FMT_VQ2, 256, 128) == 26_112
    assert _lib.expert_bytes(_lib.FMT_ABSENT, 256, 128) == 0
    assert _lib.expert_bytes(_lib.FMT_VQ2, 100, 128) == 0
    assert _lib.expert_bytes(_lib.FMT_VQ2, 256, 0) == 0
    assert _lib.expert_bytes(7, 256, 128) == 0


@pytest.mark.parametrize("fmt", [_lib.FMT_VQ2, _lib.FMT_MXFP4])
@pytest.mark.parametrize("dims", [(256, 128), (7168, 2048), (384, 640)])
def test_slot_layout_matches_oracle_reading(fmt, dims):
    H, I = dims
    offs = _lib.slot_layout(fmt, H, I)
    blocks, total = oracle.slot_blocks(fmt, H, I)
    assert offs[6] == total == _lib.expert_bytes(fmt, H, I)
    assert offs[:6] == [b[3] for b in blocks]
    assert all(o % 256 == 0 for o in offs)


@pytest.mark.parametrize("fmt", [synth.FMT_VQ2, synth.FMT_MXFP4])
def test_packed_slot_reads_back(fmt):
    cfg = synth.PRESETS["tiny"]
    ex = synth.draw_expert(cfg, 2, fmt)
    buf = pack_slot(ex, cfg.hidden, cfg.inter)
    pool = np.zeros(512 + buf.size, dtype=np.uint8)
    pool[512:] = buf
    back = oracle.read_slot(pool, 512, fmt, cfg.hidden, cfg.inter)
    for key, val in ex.items():
        if key == "format":
            continue
        assert np.array_equal(back[key].view(np.uint8), np.asarray(val).view(np.uint8)), key


def test_pack_slot_refuses_arrays_of_another_format():
    # arrays of one format packed under another slot format would fill only part of
    # the slot; the packer must refuse, and the layer draws the expert in the slot's format instead
    cfg = synth.PRESETS["tiny"]
    ex = synth.draw_expert(cfg, 1, synth.FMT_VQ2)
    with pytest.raises(ValueError):
        pack_slot(ex, cfg.hidden, cfg.inter, synth.FMT_MXFP4)
    syn = synth.SynthLayer(cfg)
    for fmt in (synth.FMT_VQ2, synth.FMT_MXFP4):
        e = 1
        got = syn.expert_as(e, fmt)
        assert int(got["format"]) == fmt
        assert pack_slot(got, cfg.hidden, cfg.inter, fmt).size == _lib.expert_bytes(fmt, cfg.hidden, cfg.inter)


def fake_layer(H=256, I=128, E=8, k=2, pool=1 << 20):
    # pointer values are never dereferenced by the paths exercised here
    return _lib.Layer(H, I, E, k, 0x10000, 0x20000, 0x100000, pool, 0x30000)


def test_workspace_bytes():
    L = fake_layer()
    a = _lib.workspace_bytes(L, 4)
    b = _lib.workspace_bytes(L, 64)
    assert 0 < a < b and a % 256 == 0
    assert _lib.workspace_bytes(fake_layer(H=100), 4) == 0
    assert _lib.workspace_bytes(fake_layer(k=9), 4) == 0
    assert _lib.workspace_bytes(L, -1) == 0
    assert _lib.workspace_bytes(L, 65537) == 0


def _status(fn, *args):
    return fn(*args)


def test_route_rejects_bad_arguments_before_any_hip_call():
    raw = _lib.raw()
    L = fake_layer()
    ws_ok = _lib.workspace_bytes(L, 4)
    P = ctypes.byref
    X, IDS, W, WS = 0x40000, 0x50000, 0x60000, 0x700000
    route = raw.moe_vq_route_topk
    assert route(None, X, _lib.F32, 4, IDS, W, WS, ws_ok, None) == _lib.EINVAL
    assert route(P(fake_layer(H=100)), X, _lib.F32, 4, IDS, W, WS, ws_ok, None) == _lib.EINVAL
    assert route(P(fake_layer(I=129)), X, _lib.F32, 4, IDS, W, WS, ws_ok, None) == _lib.EINVAL
    assert route(P(fake_layer(k=9)), X, _lib.F32, 4, IDS, W, WS, ws_ok, None) == _lib.EINVAL
    assert route(P(fake_layer(E=0)), X, _lib.F32, 4, IDS, W, WS, ws_ok, None) == _lib.EINVAL
    assert route(P(L), X, 7, 4, IDS, W, WS, ws_ok, None) == _lib.EINVAL
    assert route(P(L), X, _lib.F32, -1, IDS, W, WS, ws_ok, None) == _lib.EINVAL
    assert route(P(L), X, _lib.F32, 4, IDS, W, None, ws_ok, None) == _lib.EINVAL
    assert route(P(L), X, _lib.F32, 4, IDS, W, WS + 8, ws_ok, None) == _lib.EINVAL
    assert route(P(L), X, _lib.F32, 4, IDS, W, WS, ws_ok - 1, None) == _lib.ENOSPACE
    assert route(P(L), None, _lib.F32, 4, IDS, W, WS, ws_ok, None) == _lib.EINVAL
    assert route(P(L), X, _lib.F32, 4, None, W, WS, ws_ok, None) == _lib.EINVAL
    # no tokens: a no-op that touches nothing
    assert route(P(L), X, _lib.F32, 0, IDS, W, WS, ws_ok, None) == _lib.OK
    bad_pool = _lib.Layer(256, 128, 8, 2, 0x10000, 0x20000, 0x100010, 1 << 20, 0x30000)
    assert route(P(bad_pool), X, _lib.F32, 4, IDS, W, WS, ws_ok, None) == _lib.EINVAL


def test_fc_and_prefill_and_decode_reject_bad_arguments():
    raw = _lib.raw()
    L = fake_layer()
    P = ctypes.byref
    ws_ok = _lib.workspace_bytes(L, 4)
    WS, H_, Y = 0x700000, 0x800000, 0x900000
    X = 0x40000
    assert raw.moe_vq_fc1_silu(P(L), X, _lib.F32, 4, WS, ws_ok - 256, H_, None) == _lib.ENOSPACE
    assert raw.moe_vq_fc1_silu(P(L), X, _lib.F32, 4, WS, ws_ok, None, None) == _lib.EINVAL
    assert raw.moe_vq_fc1_silu(P(L), None, _lib.F32, 4, WS, ws_ok, H_, None) == _lib.EINVAL
    assert raw.moe_vq_fc1_silu(P(L), X + 8, _lib.F32, 4, WS, ws_ok, H_, None) == _lib.EINVAL
    assert raw.moe_vq_fc1_silu(P(L), X, 9, 4, WS, ws_ok, H_, None) == _lib.EINVAL
    assert raw.moe_vq_fc1_silu(P(L), X, _lib.F32, 0, WS, ws_ok, H_, None) == _lib.OK
    assert raw.moe_vq_fc2_combine(P(L), H_, 4, WS, ws_ok, None, None) == _lib.EINVAL
    assert raw.moe_vq_fc2_combine(P(L), None, 4, WS, ws_ok, Y, None) == _lib.EINVAL
    assert raw.moe_vq_fc2_combine(P(L), H_, 4, None, ws_ok, Y, None) == _lib.EINVAL
    assert raw.moe_vq_prefill_gemm(P(L), 0x40000, 3, 4, WS, ws_ok, Y, None) == _lib.EINVAL
    assert raw.moe_vq_prefill_gemm(P(L), 0x40000, _lib.BF16, 4, WS, 0, Y, None) == _lib.ENOSPACE
    assert raw.moe_vq_decode_expert(P(L), 8, 0, _lib.F32, Y, None, None) == _lib.EINVAL
    assert raw.moe_vq_decode_expert(P(L), -1, 0, _lib.F32, Y, None, None) == _lib.EINVAL
    assert raw.moe_vq_decode_expert(P(L), 0, 3, _lib.F32, Y, None, None) == _lib.EINVAL
    assert raw.moe_vq_decode_expert(P(L), 0, 0, 5, Y, None, None) == _lib.EINVAL
    assert raw.moe_vq_decode_expert(P(L), 0, 0, _lib.F32, None, None, None) == _lib.EINVAL
    assert raw.moe_vq_check(None, None, None) == _lib.EINVAL
    assert raw.moe_vq_step_info(None, 4, WS, None, None, None) == _lib.EINVAL
    # no tokens: every step call is a no-op; more than 65536 tokens: rejected
    assert raw.moe_vq_fc2_combine(P(L), H_, 0, WS, ws_ok, Y, None) == _lib.OK
    assert raw.moe_vq_prefill_gemm(P(L), 0x40000, _lib.BF16, 0, WS, ws_ok, Y, None) == _lib.OK
    for T in (-1, 65537):
        assert raw.moe_vq_route_topk(P(L), 0x40000, _lib.F32, T, 0x50000, 0x60000, WS, ws_ok, None) == _lib.EINVAL
        assert raw.moe_vq_fc1_silu(P(L), 0x40000, _lib.F32, T, WS, ws_ok, H_, None) == _lib.EINVAL
        assert raw.moe_vq_fc2_combine(P(L), H_, T, WS, ws_ok, Y, None) == _lib.EINVAL
        assert raw.moe_vq_prefill_gemm(P(L), 0x40000, _lib.BF16, T, WS, ws_ok, Y, None) == _lib.EINVAL


def test_forward_rejects_bad_arguments():
    raw = _lib.raw()
    L = fake_layer()
    P = ctypes.byref
    ws_ok = _lib.workspace_bytes(L, 4)
    X, IDS, W, H_, Y, WS = 0x40000, 0x50000, 0x60000, 0x800000, 0x900000, 0x700000
    fwd = raw.moe_vq_forward
    assert fwd(P(L), X, _lib.BF16, 4, IDS, W, H_, Y, WS, ws_ok - 1, None) == _lib.ENOSPACE
    assert fwd(P(L), X, 5, 4, IDS, W, H_, Y, WS, ws_ok, None) == _lib.EINVAL
    assert fwd(P(L), None, _lib.BF16, 4, IDS, W, H_, Y, WS, ws_ok, None) == _lib.EINVAL
    assert fwd(P(L), X, _lib.BF16, 4, IDS, W, None, Y, WS, ws_ok, None) == _lib.EINVAL
    assert fwd(P(L), X, _lib.BF16, 4, IDS, W, H_, Y + 4, WS, ws_ok, None) == _lib.EINVAL
    assert fwd(P(L), X, _lib.BF16, 4, IDS, W, H_, Y, WS + 16, ws_ok, None) == _lib.EINVAL
    assert fwd(P(L), X, _lib.BF16, 65537, IDS, W, H_, Y, WS, ws_ok, None) == _lib.EINVAL
    assert fwd(P(L), X, _lib.BF16, 0, IDS, W, H_, Y, WS, ws_ok, None) == _lib.OK


def test_strerror():
    assert _lib.strerror(_lib.OK) == "ok"
    assert "resident" in _lib.strerror(_lib.ENOTRESIDENT)
    assert "workspace" in _lib.strerror(_lib.ENOSPACE)
    assert _lib.strerror(99) == "unknown status"


def test_single_hip_runtime_in_process():
    """The library binds the HIP runtime that PyTorch loaded (one libamdhip64 mapped),
    so torch's streams and allocations are valid for it."""
    maps = open("/proc/self/maps").read().splitlines()
    libs = sorted({ln.split()[-1] for ln in maps if "libamdhip64" in ln})
    assert len(libs) == 1, libs


def test_swiglu_limit_and_shared_expert_arguments():
    """The SwiGLU clamp's limit must be finite and >= 0 on every entry point, and the
    shared expert takes a one-expert, top-1 layer; both refused before any HIP call."""
    raw = _lib.raw()
    P = ctypes.byref
    X, IDS, W, WS, H_, Y = 0x40000, 0x50000, 0x60000, 0x700000, 0x800000, 0x900000
    for lim in (float("nan"), -1.0, float("inf")):
        L = fake_layer()
        L.swiglu_limit = lim
        ws_ok = _lib.workspace_bytes(L, 4)
        assert raw.moe_vq_route_topk(P(L), X, _lib.F32, 4, IDS, W, WS, ws_ok, None) == _lib.EINVAL
        assert raw.moe_vq_fc1_silu(P(L), X, _lib.F32, 4, WS, ws_ok, H_, None) == _lib.EINVAL
        assert raw.moe_vq_forward(P(L), X, _lib.F32, 4, IDS, W, H_, Y, WS, ws_ok, None) == _lib.EINVAL
        assert raw.moe_vq_prefill_gemm(P(L), X, _lib.F32, 4, WS, ws_ok, Y, None) == _lib.EINVAL
    S = fake_layer(E=1, k=1)
    ws_s = _lib.workspace_bytes(S, 4)
    assert ws_s > 0
    assert raw.moe_vq_shared_expert(P(fake_layer()), X, _lib.F32, 4, WS, ws_s, H_, Y, None) == _lib.EINVAL
    assert raw.moe_vq_shared_expert(P(fake_layer(E=2, k=1)), X, _lib.F32, 4, WS, ws_s, H_, Y, None) == _lib.EINVAL
    assert raw.moe_vq_shared_expert(P(S), X, _lib.F32, 4, WS, ws_s, None, Y, None) == _lib.EINVAL
    assert raw.moe_vq_shared_expert(P(S), X, _lib.F32, 4, WS, ws_s, H_, None, None) == _lib.EINVAL
    assert raw.moe_vq_shared_expert(P(S), X + 8, _lib.F32, 4, WS, ws_s, H_, Y, None) == _lib.EINVAL
    assert raw.moe_vq_shared_expert(P(S), X, 5, 4, WS, ws_s, H_, Y, None) == _lib.EINVAL
    assert raw.moe_vq_shared_expert(P(S), X, _lib.F32, 4, WS, ws_s - 256, H_, Y, None) == _lib.ENOSPACE
    assert raw.moe_vq_shared_expert(P(S), X, _lib.F32, 0, WS, ws_s, H_, Y, None) == _lib.OK
    S.swiglu_limit = float("nan")
    assert raw.moe_vq_shared_expert(P(S), X, _lib.F32, 4, WS, ws_s, H_, Y, None) == _lib.EINVAL


def test_delta_cache_arguments():
    """FP4 delta cache: its copies are listed as experts E + e, so the workspace grows;
    more than 512 experts, a negative or NaN gate, or the host miss path are refused."""
    raw = _lib.raw()
    P = ctypes.byref
    X, IDS, W, WS = 0x40000, 0x50000, 0x60000, 0x700000
    L = fake_layer(E=128)
    D = fake_layer(E=128)
    D.delta_slots, D.gate_tau = 0x38000, 0.6
    assert _lib.workspace_bytes(D, 64) > _lib.workspace_bytes(L, 64)
    ws_d = _lib.workspace_bytes(D, 4)
    assert ws_d > _lib.workspace_bytes(L, 4)
    assert raw.moe_vq_route_topk(P(D), X, _lib.F32, 0, IDS, W, WS, ws_d, None) == _lib.OK
    # the layer without the cache needs less: with the cache the smaller size is refused
    assert raw.moe_vq_route_topk(P(D), X, _lib.F32, 4, IDS, W, WS, _lib.workspace_bytes(L, 4), None) \
        == _lib.ENOSPACE
    for tau in (-0.1, float("nan"), float("inf")):
        bad = fake_layer()
        bad.delta_slots, bad.gate_tau = 0x38000, tau
        assert raw.moe_vq_route_topk(P(bad), X, _lib.F32, 0, IDS, W, WS, ws_d, None) == _lib.EINVAL
    big = fake_layer(E=513, k=2)
    big.delta_slots, big.gate_tau = 0x38000, 0.6
    assert _lib.workspace_bytes(big, 4) == 0
    assert raw.moe_vq_route_topk(P(big), X, _lib.F32, 0, IDS, W, WS, 1 << 30, None) == _lib.EINVAL
    misaligned = fake_layer()
    misaligned.delta_slots, misaligned.gate_tau = 0x38004, 0.6
    assert raw.moe_vq_route_topk(P(misaligned), X, _lib.F32, 0, IDS, W, WS, ws_d, None) == _lib.EINVAL
    Y, CMP, HP, CB = 0x90000, 0xA0000, 0xB0000, 0xD0000
    HS = (_lib.Slot * 128)()
    assert raw.moe_vq_cpu_experts(P(D), HP, 1 << 20, HS, CB, X, _lib.F32, 4, IDS, W, CMP, Y, 1) \
        == _lib.EUNSUPPORTED


def test_static_workspace_capacity_matches_its_documentation():
    """moe_vq_forward_static's 16 MiB array holds the workspace of 55 tokens at the full
    shape (H = 7168, I = 2048, 256 experts, top-8), as include/moe_vq.h states."""
    full = _lib.Layer(7168, 2048, 256, 8, 0x10000, 0x20000, 0x100000, 1 << 30, 0x30000)
    assert _lib.workspace_bytes(full, 55) <= 16 << 20 < _lib.workspace_bytes(full, 56)


def test_read_probe_rejects_bad_arguments():
    raw = _lib.raw()
    BUF, SINK = 0x100000, 0x200000
    assert raw.moe_vq_read_probe(None, 1 << 20, SINK, None) == _lib.EINVAL
    assert raw.moe_vq_read_probe(BUF, 1 << 20, None, None) == _lib.EINVAL
    assert raw.moe_vq_read_probe(BUF + 8, 1 << 20, SINK, None) == _lib.EINVAL
    assert raw.moe_vq_read_probe(BUF, (1 << 20) + 8, SINK, None) == _lib.EINVAL
    assert raw.moe_vq_read_probe(BUF, 0, SINK, None) == _lib.EINVAL
    assert raw.moe_vq_read_probe(BUF, 1 << 20, SINK + 2, None) == _lib.EINVAL
