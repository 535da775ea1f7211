"""Helpers for the GPU parity tests: device layers from the seeded generator, one
step through the C ABI, and the comparison with the fp64 oracle (the rules of the
parity contract: identical or near-tie-equivalent expert selection, routing weights
within 1e-5, per-token max |y - y_oracle| <= 1e-2 * max |y_oracle|)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import synth
from bit_vector_quantised_amd import _lib
from bit_vector_quantised_amd.layer import DeviceLayer, Step

Y_TOL = 1e-2
W_TOL = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def x_tensor(x_np: np.ndarray, x_dtype: str) -> torch.Tensor:
    if x_dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x_np).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x_np, dtype=np.float32)).cuda()


def run(dev: DeviceLayer, x_np: np.ndarray, x_dtype: str, step: Step = None):
    T = x_np.shape[0]
    st = step or Step(dev, max(T, 1))
    xt = x_tensor(x_np, x_dtype)
    st.forward(xt)
    torch.cuda.synchronize()
    status, info = st.check()
    return {
        "ids": st.ids[:T].cpu().numpy().astype(np.int64),
        "w": st.w[:T].cpu().numpy().astype(np.float64),
        "h": st.h[:T * dev.top_k].cpu().numpy().astype(np.float64).reshape(T, dev.top_k, -1),
        "y": st.y[:T].cpu().numpy().astype(np.float64),
        "status": status, "info": info, "step": st,
    }


def rel_err_rows(a: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per row: max |a - ref| / max |ref| (rows along the last axis)."""
    num = np.abs(a - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    return num / np.where(den > 0, den, 1.0)


def compare(syn, x_np: np.ndarray, x_dtype: str, g: dict, top_k: int, tokens=None, check_h=True,
            swiglu_limit=0.0, shared=None, fp4_copy=None, gate_tau=None):
    """Compare one GPU step with the oracle on the given tokens (all by default); with
    swiglu_limit / shared / fp4_copy and gate_tau, against the oracle's clamped layer /
    with its shared expert / with its FP4 delta cache."""
    x64 = oracle.x_value(x_np, x_dtype)
    T = x64.shape[0]
    tokens = list(range(T)) if tokens is None else list(tokens)
    logits = oracle.router_logits(syn.router_w, x64)
    delta = oracle.fp32_dot_error_bound(syn.router_w, x64)
    ref_ids = oracle.topk(logits, top_k)
    assert oracle.selection_is_valid(g["ids"], logits, delta, top_k), "GPU selection is not a valid top-k"
    n_diff = int((g["ids"] != ref_ids).any(axis=1).sum())
    sel = g["ids"][tokens]
    r = oracle.forward(syn, x64[tokens], top_k, forced_selection=sel, swiglu_limit=swiglu_limit, shared=shared,
                       fp4_copy=fp4_copy, gate_tau=gate_tau)
    werr = np.abs(g["w"][tokens] - r["w"]).max()
    assert werr <= W_TOL, f"routing weights off by {werr}"
    assert np.all(np.abs(g["w"].sum(axis=1) - 1.0) <= 4 * top_k * 2.0 ** -24)
    ey = rel_err_rows(g["y"][tokens], r["y"])
    assert ey.max() <= Y_TOL, f"y relative error {ey.max()}"
    eh = 0.0
    if check_h:
        eh = rel_err_rows(g["h"][tokens], r["h"]).max()
        assert eh <= Y_TOL, f"h relative error {eh}"
    return {"n_sel_diff": n_diff, "y_err": float(ey.max()), "h_err": float(eh), "w_err": float(werr),
            "ref": r}


def bf16_rne_bits(f32: np.ndarray) -> np.ndarray:
    return synth.f64_to_bf16_bits(f32.astype(np.float32))


def decode_on_gpu(dev: DeviceLayer, e: int, mat: int, out_dtype: int):
    rows = dev.hidden if mat == _lib.MAT_DOWN else dev.inter
    K = dev.inter if mat == _lib.MAT_DOWN else dev.hidden
    dt = torch.float32 if out_dtype == _lib.F32 else torch.int16
    out = torch.empty((rows, K), dtype=dt, device="cuda")
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    _lib.decode_expert(dev.c, e, mat, out_dtype, out.data_ptr(), status.data_ptr(),
                       torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return out.cpu().numpy(), int(status.item())


def run_prefill(dev: DeviceLayer, x_np: np.ndarray, x_dtype: str, step: Step = None):
    """route -> prefill grouped GEMM; returns the step's selection, weights and y."""
    T = x_np.shape[0]
    st = step or Step(dev, max(T, 1))
    xt = x_tensor(x_np, x_dtype)
    st.route(xt)
    st.prefill(xt)
    torch.cuda.synchronize()
    status, info = st.check()
    return {
        "ids": st.ids[:T].cpu().numpy().astype(np.int64),
        "w": st.w[:T].cpu().numpy().astype(np.float64),
        "y": st.y[:T].cpu().numpy().astype(np.float64),
        "status": status, "info": info, "step": st,
    }
