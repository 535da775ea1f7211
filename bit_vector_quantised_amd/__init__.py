"""MI355X-native MoE-VQ routed-expert step: a C-ABI HIP library (libmoe_vq.so,
include/moe_vq.h) and its thin Python binding.

Importing this package loads the library; it raises if the library is not built.
"""
from . import _lib  # noqa: F401  (loads libmoe_vq.so, fails loudly if missing)
from ._lib import (BF16, EHIP, EINVAL, ENOSPACE, ENOTRESIDENT, EUNSUPPORTED, F32, FMT_ABSENT,  # noqa: F401
                   FMT_MXFP4, FMT_VQ2, MAT_DOWN, MAT_GATE, MAT_UP, OK, MoeVqError, check, decode_expert,
                   expert_bytes, fc1_silu, fc2_combine, forward, prefill_gemm, route_topk, slot_layout, step_info, strerror,
                   workspace_bytes)
