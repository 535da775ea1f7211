"""Device-resident MoE-VQ layer and step buffers on top of the C ABI.

PyTorch provides device memory and the stream; every step of the computation runs
in the HIP library.  This module only places bytes (the slot pool, the slot table)
and passes pointers.
"""
from __future__ import annotations

import os
from typing import Callable, Dict, Optional, Sequence

import numpy as np
import torch

from . import _lib

PAYLOAD_KEYS = {
    _lib.FMT_VQ2: ("codes_g", "codes_u", "codes_d", "scales_g", "scales_u", "scales_d"),
    _lib.FMT_MXFP4: ("nib_g", "nib_u", "nib_d", "e8m0_g", "e8m0_u", "e8m0_d"),
}


def pack_slot(expert: Dict[str, np.ndarray], hidden: int, inter: int, fmt: Optional[int] = None) -> np.ndarray:
    """The bytes of one expert slot (layout of include/moe_vq.h, offsets from the library).
    fmt, when given, is the format the slot table will state; arrays of another format
    are refused (they would fill only part of the slot)."""
    if fmt is not None and int(fmt) != int(expert["format"]):
        raise ValueError(f"expert arrays are format {int(expert['format'])}, slot format is {int(fmt)}")
    fmt = int(expert["format"])
    offs = _lib.slot_layout(fmt, hidden, inter)
    buf = np.zeros(offs[6], dtype=np.uint8)
    for key, off in zip(PAYLOAD_KEYS[fmt], offs[:6]):
        raw = np.ascontiguousarray(expert[key]).view(np.uint8).reshape(-1)
        buf[off:off + raw.size] = raw
    return buf


def _slot_table(offsets: np.ndarray, formats: Sequence[int]) -> np.ndarray:
    slots = np.zeros(len(offsets), dtype=[("byte_offset", "<u8"), ("format", "<u4"), ("reserved", "<u4")])
    slots["byte_offset"] = offsets
    slots["format"] = np.asarray(formats, dtype=np.uint32)
    return slots


class DeviceLayer:
    """Slot pool + slot table + router weights + codebook in device memory.

    experts(e) returns expert e's storage arrays (see synth); formats[e] gives its
    format, MOE_VQ_FMT_ABSENT leaving the slot empty (not resident).  With copies (a
    function e -> storage arrays or None), the experts it returns arrays for also get an
    FP4 copy in the FP4 delta cache (the layer's delta_slots, placed after the experts in
    the same pool), used by the routed pairs whose weight reaches gate_tau.
    """

    def __init__(self, hidden: int, inter: int, n_experts: int, top_k: int, codebook: np.ndarray,
                 router_w_bits: np.ndarray, experts: Callable[[int], Dict[str, np.ndarray]],
                 formats: Sequence[int], device: str = "cuda", swiglu_limit: float = 0.0,
                 copies: Optional[Callable[[int], Optional[Dict[str, np.ndarray]]]] = None,
                 gate_tau: float = 0.0):
        self.hidden, self.inter, self.n_experts, self.top_k = hidden, inter, n_experts, top_k
        self.device = torch.device(device)
        offsets = np.zeros(n_experts, dtype=np.uint64)
        total = 0
        for e in range(n_experts):
            f = int(formats[e])
            if f == _lib.FMT_ABSENT:
                continue
            offsets[e] = total
            total += _lib.expert_bytes(f, hidden, inter)
        copy_arrays = [copies(e) for e in range(n_experts)] if copies is not None else [None] * n_experts
        copy_formats = [int(a["format"]) if a is not None else _lib.FMT_ABSENT for a in copy_arrays]
        copy_offsets = np.zeros(n_experts, dtype=np.uint64)
        for e in range(n_experts):
            if copy_arrays[e] is not None:
                copy_offsets[e] = total
                total += _lib.expert_bytes(copy_formats[e], hidden, inter)
        self.pool_bytes = max(total, 256)
        self.pool = torch.empty(self.pool_bytes, dtype=torch.uint8, device=self.device)
        for e in range(n_experts):
            f = int(formats[e])
            if f == _lib.FMT_ABSENT:
                continue
            buf = pack_slot(experts(e), hidden, inter, f)
            o = int(offsets[e])
            self.pool[o:o + buf.size].copy_(torch.from_numpy(buf))
        for e in range(n_experts):
            if copy_arrays[e] is not None:
                buf = pack_slot(copy_arrays[e], hidden, inter)
                o = int(copy_offsets[e])
                self.pool[o:o + buf.size].copy_(torch.from_numpy(buf))
        self.slot_offsets = offsets
        self.formats = np.asarray(formats, dtype=np.int32)
        self.slots = torch.from_numpy(_slot_table(offsets, formats).view(np.uint8).copy()).to(self.device)
        self.copy_formats = np.asarray(copy_formats, dtype=np.int32)
        self.delta_slots = None
        if copies is not None:
            self.delta_slots = torch.from_numpy(
                _slot_table(copy_offsets, copy_formats).view(np.uint8).copy()).to(self.device)
        self.router_w = torch.from_numpy(np.ascontiguousarray(router_w_bits).view(np.int16)).to(self.device)
        self.codebook = torch.from_numpy(np.ascontiguousarray(codebook).view(np.int16)).to(self.device)
        self.c = _lib.Layer(hidden, inter, n_experts, top_k, self.router_w.data_ptr(), self.codebook.data_ptr(),
                            self.pool.data_ptr(), self.pool_bytes, self.slots.data_ptr(), float(swiglu_limit),
                            self.delta_slots.data_ptr() if self.delta_slots is not None else None,
                            float(gate_tau))

    @classmethod
    def from_synth(cls, syn, device: str = "cuda", formats: Optional[Sequence[int]] = None,
                   swiglu_limit: float = 0.0, fp4_copies: Optional[Sequence[int]] = None,
                   gate_tau: float = 0.0):
        """fp4_copies: the experts that get an FP4 (MXFP4) copy in the delta cache."""
        cfg = syn.cfg
        fm = syn.formats if formats is None else formats
        copies = None
        if fp4_copies is not None:
            have = set(int(e) for e in fp4_copies)
            copies = lambda e: syn.expert_as(e, _lib.FMT_MXFP4) if e in have else None  # noqa: E731
        return cls(cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, syn.codebook, syn.router_w,
                   lambda e: syn.expert_as(e, fm[e]), fm, device, swiglu_limit, copies, gate_tau)

    def set_slots(self, offsets: np.ndarray, formats: Sequence[int]) -> None:
        """Rewrite the slot table (e.g. to mark experts absent)."""
        self.slots.copy_(torch.from_numpy(_slot_table(offsets, formats).view(np.uint8).copy()))


class SharedExpert:
    """The shared expert of a layer: a one-expert layer (n_experts = top_k = 1) holding its
    weights in one slot, and the buffers of moe_vq_shared_expert for up to max_tokens
    tokens.  add(x, y) adds S(x) to y [T, H] fp32 in place."""

    def __init__(self, hidden: int, inter: int, codebook: np.ndarray, expert: Dict[str, np.ndarray],
                 fmt: int, max_tokens: int, device: str = "cuda", swiglu_limit: float = 0.0):
        # (the router row is only a placeholder: one expert always has weight 1)
        self.layer = DeviceLayer(hidden, inter, 1, 1, codebook, np.zeros((1, hidden), dtype=np.uint16),
                                 lambda e: expert, [fmt], device, swiglu_limit)
        self.max_tokens = max_tokens
        self.ws_bytes = _lib.workspace_bytes(self.layer.c, max_tokens)
        if self.ws_bytes == 0:
            raise ValueError("invalid layer shape")
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.layer.device)
        self.h = torch.empty((max_tokens, inter), dtype=torch.float32, device=self.layer.device)

    def add(self, x: torch.Tensor, y: torch.Tensor) -> torch.Tensor:
        T = x.shape[0]
        assert x.is_contiguous() and x.shape[1] == self.layer.hidden and T <= self.max_tokens
        assert y.is_contiguous() and y.dtype == torch.float32 and tuple(y.shape) == (T, self.layer.hidden)
        _lib.shared_expert(self.layer.c, x.data_ptr(), x_dtype_code(x), T, self.ws.data_ptr(), self.ws_bytes,
                           self.h.data_ptr(), y.data_ptr(), torch.cuda.current_stream(self.layer.device).cuda_stream)
        return y

    def check(self):
        return _lib.check(self.ws.data_ptr(), torch.cuda.current_stream(self.layer.device).cuda_stream)


class TieredLayer:
    """A layer whose experts live in a pinned host pool, with n_dev_slots device slots
    managed by the library's expert tier (moe_vq_tier_*): the device slot table starts
    all-absent and tiered_forward() copies the experts a step selects into device slots
    (least recently used out).  Same interface as DeviceLayer for Step."""

    def __init__(self, hidden: int, inter: int, n_experts: int, top_k: int, codebook: np.ndarray,
                 router_w_bits: np.ndarray, experts: Callable[[int], Dict[str, np.ndarray]],
                 formats: Sequence[int], n_dev_slots: int, device: str = "cuda"):
        self.hidden, self.inter, self.n_experts, self.top_k = hidden, inter, n_experts, top_k
        self.device = torch.device(device)
        host_slots, total = [], 0
        for e in range(n_experts):
            f = int(formats[e])
            host_slots.append((total, f))
            if f != _lib.FMT_ABSENT:
                total += _lib.expert_bytes(f, hidden, inter)
        self.host_pool = torch.empty(max(total, 256), dtype=torch.uint8, pin_memory=True)
        for e in range(n_experts):
            o, f = host_slots[e]
            if f != _lib.FMT_ABSENT:
                buf = pack_slot(experts(e), hidden, inter, f)
                self.host_pool[o:o + buf.size].copy_(torch.from_numpy(buf))
        slot_bytes = max(_lib.expert_bytes(_lib.FMT_VQ2, hidden, inter), _lib.expert_bytes(_lib.FMT_MXFP4, hidden, inter))
        slot_bytes = (slot_bytes + 255) // 256 * 256
        self.pool_bytes = slot_bytes * n_dev_slots
        self.pool = torch.empty(self.pool_bytes, dtype=torch.uint8, device=self.device)
        self.slots = torch.zeros(n_experts * 16, dtype=torch.uint8, device=self.device)
        self.router_w = torch.from_numpy(np.ascontiguousarray(router_w_bits).view(np.int16)).to(self.device)
        self.codebook = torch.from_numpy(np.ascontiguousarray(codebook).view(np.int16)).to(self.device)
        self.codebook_host = torch.from_numpy(np.ascontiguousarray(codebook).view(np.int16).copy())
        self.host_formats = [f for _, f in host_slots]
        self.c = _lib.Layer(hidden, inter, n_experts, top_k, self.router_w.data_ptr(), self.codebook.data_ptr(),
                            self.pool.data_ptr(), self.pool_bytes, self.slots.data_ptr())
        self.readback = torch.empty(64 + n_experts, dtype=torch.int32, pin_memory=True)
        self.tier = _lib.ExpertTier(n_experts, self.host_pool.data_ptr(), host_slots,
                                    [s * slot_bytes for s in range(n_dev_slots)], self.readback.data_ptr())
        _lib.tier_init(self.c, self.tier, self.slots.data_ptr(), torch.cuda.current_stream(self.device).cuda_stream)

    @classmethod
    def from_synth(cls, syn, n_dev_slots: int, device: str = "cuda", formats: Optional[Sequence[int]] = None):
        cfg = syn.cfg
        fm = syn.formats if formats is None else formats
        return cls(cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, syn.codebook, syn.router_w,
                   lambda e: syn.expert_as(e, fm[e]), fm, n_dev_slots, device)


def tiered_forward(step: "Step", layer: TieredLayer, x: torch.Tensor):
    """route -> copy the missing experts -> (route again) -> FC1 -> FC2.  Returns
    (y view [T, H], number of experts copied)."""
    T = x.shape[0]
    step.route(x)
    n = _lib.tier_resolve(layer.c, layer.tier, layer.pool.data_ptr(), layer.slots.data_ptr(), T,
                          step.ws.data_ptr(), step.stream())
    if n:
        step.route(x)
    step.fc1(x)
    step.fc2(T)
    return step.y[:T], n


def cpu_miss_forward(step: "Step", layer: TieredLayer, x: torch.Tensor, n_threads: Optional[int] = None):
    """One step with the CPU miss path: route on the GPU; the selected experts that hold a
    device slot run on the GPU (FC1, FC2), and at the same time the host cores compute the
    others from the tier's host pool (moe_vq_cpu_experts); y is the sum.  No expert is
    copied.  Returns (y view [T, H] on the device, list of experts computed on the host).
    The GPU step's status reports the lowest expert it left out, which the host computed."""
    T = x.shape[0]
    step.route(x)
    ids = step.ids[:T].cpu()  # (synchronises the stream: the routing is needed here)
    w = step.w[:T].cpu()
    x_host = x.cpu()
    held = set(e for e in layer.tier.held() if e >= 0)
    miss = sorted(set(int(e) for e in ids.reshape(-1).tolist()) - held)
    step.fc1(x)
    step.fc2(T)  # (asynchronous: the host computes its experts meanwhile)
    y_host = torch.zeros((T, layer.hidden), dtype=torch.float32)
    if miss:
        compute = torch.zeros(layer.n_experts, dtype=torch.uint8)
        compute[miss] = 1
        threads = n_threads or max(1, min(64, len(os.sched_getaffinity(0))))
        _lib.cpu_experts(layer.c, layer.host_pool.data_ptr(), layer.host_pool.numel(), layer.tier._host_slots,
                         layer.codebook_host.data_ptr(), x_host.data_ptr(), x_dtype_code(x), T, ids.data_ptr(),
                         w.data_ptr(), compute.data_ptr(), y_host.data_ptr(), threads)
        step.y[:T].add_(y_host.to(layer.device))
    return step.y[:T], miss


def x_dtype_code(x: torch.Tensor) -> int:
    if x.dtype == torch.bfloat16:
        return _lib.BF16
    if x.dtype == torch.float32:
        return _lib.F32
    raise TypeError(f"activations must be bf16 or fp32, got {x.dtype}")


class Step:
    """Buffers for one routed-expert step of up to max_tokens tokens, and the calls."""

    def __init__(self, layer: DeviceLayer, max_tokens: int):
        self.layer = layer
        self.max_tokens = max_tokens
        dev = layer.device
        k, H, I = layer.top_k, layer.hidden, layer.inter
        self.ws_bytes = _lib.workspace_bytes(layer.c, max_tokens)
        if self.ws_bytes == 0:
            raise ValueError("invalid layer shape")
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.ids = torch.empty((max_tokens, k), dtype=torch.int32, device=dev)
        self.w = torch.empty((max_tokens, k), dtype=torch.float32, device=dev)
        self.h = torch.empty((max_tokens * k, I), dtype=torch.float32, device=dev)
        self.y = torch.empty((max_tokens, H), dtype=torch.float32, device=dev)

    def stream(self) -> int:
        return torch.cuda.current_stream(self.layer.device).cuda_stream

    def route(self, x: torch.Tensor) -> None:
        T = x.shape[0]
        assert x.is_contiguous() and x.shape[1] == self.layer.hidden and T <= self.max_tokens
        _lib.route_topk(self.layer.c, x.data_ptr(), x_dtype_code(x), T, self.ids.data_ptr(), self.w.data_ptr(),
                        self.ws.data_ptr(), self.ws_bytes, self.stream())

    def fc1(self, x: torch.Tensor) -> None:
        """FC1 of the step routed on x (the same tensor route() was given)."""
        _lib.fc1_silu(self.layer.c, x.data_ptr(), x_dtype_code(x), x.shape[0], self.ws.data_ptr(), self.ws_bytes,
                      self.h.data_ptr(), self.stream())

    def fc2(self, T: int) -> None:
        _lib.fc2_combine(self.layer.c, self.h.data_ptr(), T, self.ws.data_ptr(), self.ws_bytes,
                         self.y.data_ptr(), self.stream())

    def prefill(self, x: torch.Tensor) -> None:
        T = x.shape[0]
        _lib.prefill_gemm(self.layer.c, x.data_ptr(), x_dtype_code(x), T, self.ws.data_ptr(), self.ws_bytes,
                          self.y.data_ptr(), self.stream())

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        """route -> FC1 -> FC2 as three calls; returns a view of y [T, H] (valid until the
        next call)."""
        T = x.shape[0]
        self.route(x)
        self.fc1(x)
        self.fc2(T)
        return self.y[:T]

    def step(self, x: torch.Tensor) -> torch.Tensor:
        """The same step through the single-call entry point moe_vq_forward."""
        T = x.shape[0]
        assert x.is_contiguous() and x.shape[1] == self.layer.hidden and T <= self.max_tokens
        _lib.forward(self.layer.c, x.data_ptr(), x_dtype_code(x), T, self.ids.data_ptr(), self.w.data_ptr(),
                     self.h.data_ptr(), self.y.data_ptr(), self.ws.data_ptr(), self.ws_bytes, self.stream())
        return self.y[:T]

    def check(self):
        return _lib.check(self.ws.data_ptr(), self.stream())

    def info(self, T: int):
        return _lib.step_info(self.layer.c, T, self.ws.data_ptr(), self.stream())
