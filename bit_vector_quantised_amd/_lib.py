"""ctypes binding of libmoe_vq.so (include/moe_vq.h): argument marshalling only.

Every function has the C entry point's name without the ``moe_vq_`` prefix, takes
device pointers as Python ints and raises MoeVqError on a nonzero status.  The
library is loaded from this package's directory; if it is missing the import fails
loudly -- there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_vq.so")

OK, EINVAL, EUNSUPPORTED, ENOSPACE, EHIP, ENOTRESIDENT = range(6)
F32, BF16 = 0, 1
FMT_ABSENT, FMT_VQ2, FMT_MXFP4 = 0, 1, 2
MAT_GATE, MAT_UP, MAT_DOWN = 0, 1, 2

EXPORTS = ("moe_vq_expert_bytes", "moe_vq_slot_layout", "moe_vq_workspace_bytes", "moe_vq_route_topk",
           "moe_vq_fc1_silu", "moe_vq_fc2_combine", "moe_vq_forward", "moe_vq_forward_static", "moe_vq_shared_expert", "moe_vq_prefill_gemm", "moe_vq_decode_expert",
           "moe_vq_check", "moe_vq_step_info", "moe_vq_tier_init", "moe_vq_tier_plan", "moe_vq_tier_resolve", "moe_vq_cpu_experts",
           "moe_vq_time_next_kernel", "moe_vq_read_probe", "moe_vq_last_hip_error", "moe_vq_strerror")


class MoeVqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        extra = f": {last_hip_error()}" if status == EHIP else ""
        super().__init__(f"{where}: status {status} ({strerror(status)}{extra})")


class Slot(ctypes.Structure):
    _fields_ = [("byte_offset", ctypes.c_uint64), ("format", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]


class Layer(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("router_w", ctypes.c_void_p), ("codebook", ctypes.c_void_p),
                ("pool", ctypes.c_void_p), ("pool_bytes", ctypes.c_uint64), ("slots", ctypes.c_void_p),
                ("swiglu_limit", ctypes.c_float), ("delta_slots", ctypes.c_void_p), ("gate_tau", ctypes.c_float)]


class Tier(ctypes.Structure):
    _fields_ = [("host_pool", ctypes.c_void_p), ("host_slots", ctypes.POINTER(Slot)), ("n_dev_slots", ctypes.c_int32),
                ("dev_slot_offsets", ctypes.POINTER(ctypes.c_uint64)),
                ("dev_slot_expert", ctypes.POINTER(ctypes.c_int32)),
                ("dev_slot_stamp", ctypes.POINTER(ctypes.c_uint64)), ("slot_mirror", ctypes.POINTER(Slot)),
                ("step", ctypes.c_uint64), ("readback", ctypes.c_void_p)]


def _load():
    # The library must run on the same HIP runtime as PyTorch, whose streams and
    # device memory it is handed.  The torch wheel bundles libamdhip64.so.7 under the
    # same soname as the system ROCm; loading torch first makes the dynamic linker
    # bind this library to torch's copy instead of starting a second runtime.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python bit_vector_quantised_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH, mode=ctypes.RTLD_GLOBAL)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    LP = ctypes.POINTER(Layer)
    sig = {
        "moe_vq_expert_bytes": (sz, [i32, i32, i32]),
        "moe_vq_slot_layout": (i32, [i32, i32, i32, ctypes.POINTER(ctypes.c_uint64)]),
        "moe_vq_workspace_bytes": (sz, [LP, i32]),
        "moe_vq_route_topk": (i32, [LP, vp, i32, i32, vp, vp, vp, sz, vp]),
        "moe_vq_fc1_silu": (i32, [LP, vp, i32, i32, vp, sz, vp, vp]),
        "moe_vq_fc2_combine": (i32, [LP, vp, i32, vp, sz, vp, vp]),
        "moe_vq_forward": (i32, [LP, vp, i32, i32, vp, vp, vp, vp, vp, sz, vp]),
        "moe_vq_forward_static": (i32, [LP, vp, i32, i32, vp, vp, vp, vp, vp, vp]),
        "moe_vq_shared_expert": (i32, [LP, vp, i32, i32, vp, sz, vp, vp, vp]),
        "moe_vq_prefill_gemm": (i32, [LP, vp, i32, i32, vp, sz, vp, vp]),
        "moe_vq_decode_expert": (i32, [LP, i32, i32, i32, vp, vp, vp]),
        "moe_vq_check": (i32, [vp, vp, ctypes.POINTER(ctypes.c_int32)]),
        "moe_vq_step_info": (i32, [LP, i32, vp, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32), vp]),
        "moe_vq_tier_init": (i32, [LP, ctypes.POINTER(Tier), vp, vp]),
        "moe_vq_tier_plan": (i32, [ctypes.POINTER(Tier), i32, ctypes.POINTER(ctypes.c_int32), i32,
                                   ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32),
                                   ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int)]),
        "moe_vq_tier_resolve": (i32, [LP, ctypes.POINTER(Tier), vp, vp, i32, vp, vp, ctypes.POINTER(ctypes.c_int32)]),
        "moe_vq_cpu_experts": (i32, [LP, vp, ctypes.c_uint64, ctypes.POINTER(Slot), vp, vp, i32, i32, vp, vp, vp,
                                     vp, i32]),
        "moe_vq_time_next_kernel": (i32, [vp, vp]),
        "moe_vq_read_probe": (i32, [vp, sz, vp, vp]),
        "moe_vq_last_hip_error": (ctypes.c_char_p, []),
        "moe_vq_strerror": (ctypes.c_char_p, [i32]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()


def _ok(status: int, where: str) -> None:
    if status != OK:
        raise MoeVqError(status, where)


def time_next_kernel(start_event: int, stop_event: int) -> None:
    """The next FC kernel launched from this thread records the two events (raw hipEvent_t
    handles, e.g. torch.cuda.Event(enable_timing=True).cuda_event) at its start and end."""
    _ok(_lib.moe_vq_time_next_kernel(start_event or None, stop_event or None), "time_next_kernel")


def read_probe(buf: int, nbytes: int, sink: int, stream: int = 0) -> None:
    """Enqueue a plain streaming read of nbytes at buf (a measurement of the read rate)."""
    _ok(_lib.moe_vq_read_probe(buf, nbytes, sink, stream), "read_probe")


def last_hip_error() -> str:
    return _lib.moe_vq_last_hip_error().decode()


def strerror(status: int) -> str:
    return _lib.moe_vq_strerror(int(status)).decode()


def expert_bytes(fmt: int, hidden: int, inter: int) -> int:
    return int(_lib.moe_vq_expert_bytes(fmt, hidden, inter))


def slot_layout(fmt: int, hidden: int, inter: int):
    off = (ctypes.c_uint64 * 7)()
    _ok(_lib.moe_vq_slot_layout(fmt, hidden, inter, off), "slot_layout")
    return [int(v) for v in off]


def workspace_bytes(layer: Layer, n_tokens: int) -> int:
    return int(_lib.moe_vq_workspace_bytes(ctypes.byref(layer), n_tokens))


def route_topk(layer: Layer, x: int, x_dtype: int, n_tokens: int, topk_ids: int, topk_w: int,
               ws: int, ws_bytes: int, stream: int = 0) -> None:
    _ok(_lib.moe_vq_route_topk(ctypes.byref(layer), x, x_dtype, n_tokens, topk_ids, topk_w, ws, ws_bytes,
                               stream), "route_topk")


def fc1_silu(layer: Layer, x: int, x_dtype: int, n_tokens: int, ws: int, ws_bytes: int, h: int,
             stream: int = 0) -> None:
    _ok(_lib.moe_vq_fc1_silu(ctypes.byref(layer), x, x_dtype, n_tokens, ws, ws_bytes, h, stream), "fc1_silu")


def fc2_combine(layer: Layer, h: int, n_tokens: int, ws: int, ws_bytes: int, y: int, stream: int = 0) -> None:
    _ok(_lib.moe_vq_fc2_combine(ctypes.byref(layer), h, n_tokens, ws, ws_bytes, y, stream), "fc2_combine")


def forward(layer: Layer, x: int, x_dtype: int, n_tokens: int, topk_ids: int, topk_w: int, h: int, y: int,
            ws: int, ws_bytes: int, stream: int = 0) -> None:
    _ok(_lib.moe_vq_forward(ctypes.byref(layer), x, x_dtype, n_tokens, topk_ids, topk_w, h, y, ws, ws_bytes,
                            stream), "forward")


def forward_static(layer: Layer, x: int, x_dtype: int, n_tokens: int, topk_ids: int, topk_w: int, h: int,
                   y: int, status: int = 0, stream: int = 0) -> None:
    _ok(_lib.moe_vq_forward_static(ctypes.byref(layer), x, x_dtype, n_tokens, topk_ids, topk_w, h, y, status,
                                   stream), "forward_static")


def shared_expert(layer: Layer, x: int, x_dtype: int, n_tokens: int, ws: int, ws_bytes: int, h: int, y: int,
                  stream: int = 0) -> None:
    _ok(_lib.moe_vq_shared_expert(ctypes.byref(layer), x, x_dtype, n_tokens, ws, ws_bytes, h, y, stream),
        "shared_expert")


def prefill_gemm(layer: Layer, x: int, x_dtype: int, n_tokens: int, ws: int, ws_bytes: int, y: int,
                 stream: int = 0) -> None:
    _ok(_lib.moe_vq_prefill_gemm(ctypes.byref(layer), x, x_dtype, n_tokens, ws, ws_bytes, y, stream),
        "prefill_gemm")


def decode_expert(layer: Layer, expert: int, matrix: int, out_dtype: int, out: int, status_dev: int = 0,
                  stream: int = 0) -> None:
    _ok(_lib.moe_vq_decode_expert(ctypes.byref(layer), expert, matrix, out_dtype, out, status_dev, stream),
        "decode_expert")


def check(ws: int, stream: int = 0):
    """(status, info) of the last step on ws; synchronises the stream."""
    info = ctypes.c_int32(-1)
    st = _lib.moe_vq_check(ws, stream, ctypes.byref(info))
    if st in (EINVAL, EHIP) and ws == 0:
        raise MoeVqError(st, "check")
    return int(st), int(info.value)


def step_info(layer: Layer, n_tokens: int, ws: int, stream: int = 0):
    """dict(status, info, n_active, n_pairs, experts) of the last step on ws; synchronises."""
    summ = (ctypes.c_int32 * 4)()
    ex = (ctypes.c_int32 * max(1, layer.n_experts * (2 if layer.delta_slots else 1)))()
    _ok(_lib.moe_vq_step_info(ctypes.byref(layer), n_tokens, ws, summ, ex, stream), "step_info")
    n = int(summ[2])
    return {"status": int(summ[0]), "info": int(summ[1]), "n_active": n, "n_pairs": int(summ[3]),
            "experts": [int(v) for v in ex[:n]]}


class ExpertTier:
    """Caller-owned state of a host-RAM expert tier (struct moe_vq_tier): keeps the
    host arrays the C structure points to alive.  host_pool: address of a pinned host
    buffer holding every expert's slot; host_slots: [(byte_offset, format)] per expert;
    dev_slot_offsets: offsets in the device pool of the slots the tier manages;
    readback: address of a pinned host buffer of 64 + n_experts 32-bit words, or 0."""

    def __init__(self, n_experts: int, host_pool: int, host_slots, dev_slot_offsets, readback: int = 0):
        self.n_experts = n_experts
        self._host_slots = (Slot * n_experts)(*[Slot(int(o), int(f), 0) for o, f in host_slots])
        ns = len(dev_slot_offsets)
        self._offs = (ctypes.c_uint64 * ns)(*[int(o) for o in dev_slot_offsets])
        self._held = (ctypes.c_int32 * ns)(*([-1] * ns))
        self._stamp = (ctypes.c_uint64 * ns)()
        self._mirror = (Slot * n_experts)()
        self.c = Tier(host_pool, self._host_slots, ns, self._offs, self._held, self._stamp, self._mirror, 0,
                      readback or None)

    def held(self):
        """Expert held by each device slot (-1 = free)."""
        return [int(v) for v in self._held]

    def stamps(self):
        return [int(v) for v in self._stamp]

    def set_state(self, held, stamps):
        """Overwrite the slot state (for exercising the plan on the host)."""
        for i, (h, t) in enumerate(zip(held, stamps)):
            self._held[i] = int(h)
            self._stamp[i] = int(t)


def tier_init(layer: Layer, tier: ExpertTier, slots: int, stream: int = 0) -> None:
    _ok(_lib.moe_vq_tier_init(ctypes.byref(layer), ctypes.byref(tier.c), slots, stream), "tier_init")


def tier_plan(tier: ExpertTier, active):
    """[(expert, device slot, evicted expert or -1)] for a step selecting `active`."""
    n = len(active)
    act = (ctypes.c_int32 * max(1, n))(*active)
    ie, isl, ev = ((ctypes.c_int32 * max(1, n))() for _ in range(3))
    cnt = ctypes.c_int(0)
    _ok(_lib.moe_vq_tier_plan(ctypes.byref(tier.c), tier.n_experts, act, n, ie, isl, ev, ctypes.byref(cnt)),
        "tier_plan")
    return [(int(ie[i]), int(isl[i]), int(ev[i])) for i in range(cnt.value)]


def tier_resolve(layer: Layer, tier: ExpertTier, pool: int, slots: int, n_tokens: int, ws: int,
                 stream: int = 0) -> int:
    """Copy the missing experts of the step last routed on ws; returns how many (route
    again before FC1 if not 0).  Synchronises stream."""
    n = ctypes.c_int32(0)
    _ok(_lib.moe_vq_tier_resolve(ctypes.byref(layer), ctypes.byref(tier.c), pool, slots, n_tokens, ws, stream,
                                 ctypes.byref(n)), "tier_resolve")
    return int(n.value)


def cpu_experts(layer: Layer, host_pool: int, host_pool_bytes: int, host_slots, codebook: int, x: int,
                x_dtype: int, n_tokens: int, topk_ids: int, topk_w: int, compute: int, y: int, n_threads: int) -> None:
    """The CPU miss path (host pointers only); host_slots is a ctypes Slot array."""
    _ok(_lib.moe_vq_cpu_experts(ctypes.byref(layer), host_pool, host_pool_bytes, host_slots, codebook, x, x_dtype,
                                n_tokens, topk_ids, topk_w, compute, y, n_threads), "cpu_experts")


def raw():
    """The loaded ctypes library (for symbol checks)."""
    return _lib
