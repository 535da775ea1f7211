"""Seeded synthetic inputs for the MoE-VQ routed-expert step.

This module is shared by the fp64 oracle (``oracle/``) and the HIP path's tests and
bench.  It holds random draws and the rounding of those draws into the storage
dtypes (fp16, bf16, u8) only.  None of the method's arithmetic lives here: no
codebook decode, no router product, no softmax/top-k, no MLP.

Workloads (shapes and distributions) follow the five synthetic configurations of
the routed-expert step: a tiny layer, decode batch 1, decode batch 32 with a
Zipf(1.1) expert popularity, batch 8 with the 52 most-routed experts kept as
MXFP4, and a 4096-token prefill chunk.  Every array is drawn from a numpy PCG64
stream keyed by (seed, purpose, index), so one expert can be regenerated without
drawing the others.

Storage formats produced (byte-exact contract with the library):
  codebook   fp16 [128, 4]          ~N(0,1), redrawn until no entry is the zero
                                    vector and no two entries are equal up to sign
  router_w   bf16 bits u16 [E, H]   ~N(0, 0.02)
  VQ2 expert codes_{g,u} u8 [I, H/4], codes_d u8 [H, I/4]   uniform bytes
             scales_{g,u} fp16 [I, H/128], scales_d fp16 [H, I/128]  ~U(0.005, 0.02)
  MXFP4 expert nib_{g,u} u8 [I, H/2], nib_d u8 [H, I/2]     uniform bytes
             e8m0_{g,u} u8 [I, H/32], e8m0_d u8 [H, I/32]    uniform over {118,119,120}
  x          fp32 [T, H] (tiny) or bf16 bits u16 [T, H]
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Dict, List, Optional

import numpy as np

FMT_ABSENT = 0
FMT_VQ2 = 1
FMT_MXFP4 = 2


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    n_tokens: int
    hidden: int
    inter: int
    n_experts: int
    top_k: int
    x_dtype: str            # "f32" or "bf16"
    routing: str            # "normal" (x ~ N(0,1)) or "zipf" (logits drawn with Zipf popularity)
    zipf_s: float = 1.1
    n_mxfp4: int = 0        # the n most popular experts (Zipf rank) are stored as MXFP4
    seed: int = 0


PRESETS: Dict[str, Config] = {
    "tiny": Config("tiny", 4, 256, 128, 8, 2, "f32", "normal", seed=1001),
    "b1": Config("b1", 1, 7168, 2048, 256, 8, "bf16", "normal", seed=1002),
    "b32": Config("b32", 32, 7168, 2048, 256, 8, "bf16", "zipf", seed=1003),
    "b8mx": Config("b8mx", 8, 7168, 2048, 256, 8, "bf16", "zipf", n_mxfp4=52, seed=1004),
    "p4096": Config("p4096", 4096, 7168, 2048, 256, 8, "bf16", "normal", seed=1005),
}


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


# ---- storage rounding (data preparation, not method arithmetic) -------------------

def f64_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round to bf16 (round-to-nearest-even via fp32) and return the u16 bit patterns."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---- draws -------------------------------------------------------------------------

def draw_codebook(seed: int) -> np.ndarray:
    """fp16 [128, 4] ~N(0,1); redrawn until the entries are pairwise distinct up to
    sign and none is the zero vector, so that the signed 256-word codebook has 256
    distinct words."""
    for attempt in range(1000):
        cb = _rng(seed, 0, attempt).standard_normal((128, 4)).astype(np.float16)
        rows = [tuple(r.view(np.uint16).tolist()) for r in cb]
        neg = [tuple((-r).view(np.uint16).tolist()) for r in cb]
        zero = any(np.all(r == 0) for r in cb.astype(np.float64))
        if not zero and len(set(rows) | set(neg)) == 256:
            return cb
    raise RuntimeError("could not draw a non-degenerate codebook")


def draw_router(cfg: Config, seed: Optional[int] = None) -> np.ndarray:
    s = cfg.seed if seed is None else seed
    w = _rng(s, 2).standard_normal((cfg.n_experts, cfg.hidden)) * 0.02
    return f64_to_bf16_bits(w)


def zipf_rank(cfg: Config, seed: Optional[int] = None) -> np.ndarray:
    """rank[e] in [0, E): popularity rank of expert e (0 = most popular)."""
    s = cfg.seed if seed is None else seed
    perm = _rng(s, 4).permutation(cfg.n_experts)
    rank = np.empty(cfg.n_experts, dtype=np.int64)
    rank[perm] = np.arange(cfg.n_experts)
    return rank


def expert_formats(cfg: Config, seed: Optional[int] = None) -> np.ndarray:
    fm = np.full(cfg.n_experts, FMT_VQ2, dtype=np.int32)
    if cfg.n_mxfp4 > 0:
        rank = zipf_rank(cfg, seed)
        fm[rank < cfg.n_mxfp4] = FMT_MXFP4
    return fm


def draw_expert(cfg: Config, e: int, fmt: int, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Arrays of expert e in its storage format (see the module docstring)."""
    s = cfg.seed if seed is None else seed
    H, I = cfg.hidden, cfg.inter
    rng = _rng(s, 1, e)
    out: Dict[str, np.ndarray] = {"format": np.int32(fmt)}
    if fmt == FMT_VQ2:
        out["codes_g"] = rng.integers(0, 256, (I, H // 4), dtype=np.uint8)
        out["codes_u"] = rng.integers(0, 256, (I, H // 4), dtype=np.uint8)
        out["codes_d"] = rng.integers(0, 256, (H, I // 4), dtype=np.uint8)
        out["scales_g"] = rng.uniform(0.005, 0.02, (I, H // 128)).astype(np.float16)
        out["scales_u"] = rng.uniform(0.005, 0.02, (I, H // 128)).astype(np.float16)
        out["scales_d"] = rng.uniform(0.005, 0.02, (H, I // 128)).astype(np.float16)
    elif fmt == FMT_MXFP4:
        out["nib_g"] = rng.integers(0, 256, (I, H // 2), dtype=np.uint8)
        out["nib_u"] = rng.integers(0, 256, (I, H // 2), dtype=np.uint8)
        out["nib_d"] = rng.integers(0, 256, (H, I // 2), dtype=np.uint8)
        out["e8m0_g"] = rng.integers(118, 121, (I, H // 32), dtype=np.uint8)
        out["e8m0_u"] = rng.integers(118, 121, (I, H // 32), dtype=np.uint8)
        out["e8m0_d"] = rng.integers(118, 121, (H, I // 32), dtype=np.uint8)
    else:
        raise ValueError(f"unknown format {fmt}")
    return out


def _x_normal(cfg: Config, n: int, stream: int, seed: int) -> np.ndarray:
    return _rng(seed, 3, stream).standard_normal((n, cfg.hidden))


def _x_zipf(cfg: Config, router_bits: np.ndarray, n: int, stream: int, seed: int) -> np.ndarray:
    """Activations whose router logits follow a Zipf(s) expert popularity.

    Target logits l*[t, e] = ln p[rank(e)] + G[t, e] with p_r proportional to
    (r+1)^-s and G ~ Gumbel(0, 1); the k largest of such logits form a sample of
    k experts without replacement with probabilities p (Gumbel-top-k).  x is the
    minimum-norm solution of W_r x = l* plus a N(0,1) component orthogonal to the
    rows of W_r, so x stays roughly N(0,1) and the router is an ordinary product.
    This is a least-squares solve for input shaping, done in fp64 before x is
    rounded to its storage dtype.
    """
    rank = zipf_rank(cfg, seed)
    p = (np.arange(cfg.n_experts, dtype=np.float64) + 1.0) ** (-cfg.zipf_s)
    p /= p.sum()
    rng = _rng(seed, 5, stream)
    gum = rng.gumbel(0.0, 1.0, (n, cfg.n_experts))
    target = np.log(p[rank])[None, :] + gum                      # [n, E]
    W = bf16_bits_to_f32(router_bits).astype(np.float64)          # [E, H]
    G = W @ W.T
    a = np.linalg.solve(G, target.T)                              # [E, n]
    x_par = (W.T @ a).T                                           # [n, H]
    z = rng.standard_normal((n, cfg.hidden))
    z_perp = z - (W.T @ np.linalg.solve(G, W @ z.T)).T
    return x_par + z_perp


def draw_x(cfg: Config, n: Optional[int] = None, stream: int = 0,
           router_bits: Optional[np.ndarray] = None, seed: Optional[int] = None) -> np.ndarray:
    """n tokens of activations in the storage dtype (fp32 array, or u16 bf16 bits)."""
    s = cfg.seed if seed is None else seed
    n = cfg.n_tokens if n is None else n
    if cfg.routing == "zipf":
        if router_bits is None:
            router_bits = draw_router(cfg, s)
        x = _x_zipf(cfg, router_bits, n, stream, s)
    else:
        x = _x_normal(cfg, n, stream, s)
    if cfg.x_dtype == "f32":
        return x.astype(np.float32)
    return f64_to_bf16_bits(x)


class SynthLayer:
    """A seeded synthetic MoE-VQ layer.  Experts are drawn on first use and cached."""

    def __init__(self, cfg: Config, seed: Optional[int] = None, cache: bool = True):
        self.cfg = cfg
        self.seed = cfg.seed if seed is None else seed
        self.codebook = draw_codebook(self.seed)
        self.router_w = draw_router(cfg, self.seed)
        self.formats = expert_formats(cfg, self.seed)
        self._cache: Dict[int, Dict[str, np.ndarray]] = {}
        self._use_cache = cache

    def expert(self, e: int) -> Dict[str, np.ndarray]:
        if e in self._cache:
            return self._cache[e]
        a = draw_expert(self.cfg, e, int(self.formats[e]), self.seed)
        if self._use_cache:
            self._cache[e] = a
        return a

    def expert_as(self, e: int, fmt: int) -> Dict[str, np.ndarray]:
        """Expert e stored in format fmt (its drawn format when fmt matches it)."""
        if int(fmt) == int(self.formats[e]):
            return self.expert(e)
        return draw_expert(self.cfg, e, int(fmt), self.seed)

    def x(self, n: Optional[int] = None, stream: int = 0) -> np.ndarray:
        return draw_x(self.cfg, n, stream, self.router_w, self.seed)

    def fingerprint(self, experts: Optional[List[int]] = None) -> str:
        h = hashlib.sha256()
        h.update(self.codebook.tobytes())
        h.update(self.router_w.tobytes())
        for e in (experts if experts is not None else range(self.cfg.n_experts)):
            a = self.expert(e)
            for k in sorted(a):
                h.update(np.asarray(a[k]).tobytes())
        return h.hexdigest()[:16]
