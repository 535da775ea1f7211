"""Plain, slow fp64 oracle of the MoE-VQ routed-expert step (test infrastructure).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use it.
It shares no code with the HIP library and is never on the product path.

What is computed, and where it comes from
-----------------------------------------
Sources are the three pages of the reference text, cited by page and section:
  [Tandem]  Tandem-vLLM 0.2.0 announcement -- sections "How it works",
            "Quality vs the official FP4 checkpoint".
  [Moet]    "vLLM-Moet: frontier MoE models on consumer/workstation Blackwell
            (SM120)" -- sections "2-bit experts on vLLM v0.24.0", "What we
            changed against official vLLM" (row "MoE at decode"),
            "Qwen3.8-Flash-Next-FP8 on 4x RTX PRO 6000", "Quality vs native".
The pages name the method but do not print its formulas; the storage format of
the synthetic workload fixes the rest (an 8-bit word = 1 sign bit + a 7-bit index
into a per-layer 128x4 fp16 codebook, one fp16 scale per 128 weights; routing is a
softmax over the router logits, top-k, renormalised).  Readings taken where both
are silent are listed next to each function (R1..R12) and in the design notes.

  O1  VQ2 decode      W[n, 4j+d] = S[n, (4j+d) // 128] * sgn(b) * CB[b & 0x7F, d],
                      b = codes[n, j], sgn(b) = -1 if b & 0x80 else +1.
                      [Tandem "How it works": experts stored as 2-bit vector codes,
                      about 2.1 bits/weight; Moet "2-bit experts": the codebook is
                      sign-symmetric.]
  O1' MXFP4 decode    W[n, k] = E2M1(q) * 2^(e - 127), q the k-th 4-bit element
                      (low nibble first), e the E8M0 exponent of k's block of 32.
                      [Tandem "Quality": the most-routed experts kept in the
                      original FP4; Moet: the official experts are MXFP4; value
                      table from the OCP Microscaling Formats v1.0 spec.]
  O2  router          l[t, e] = sum_h W_r[e, h] x[t, h]
  O3  softmax         p = exp(l - max l) / sum exp(l - max l)
  O4  top-k           the k largest logits, by descending logit, ties -> lower id
  O5  renormalise     w_i = p[S_i] / sum_{j in S} p[j]
  O6  FC1 + SiLU*up   g = W_g x, u = W_u x, h = g / (1 + exp(-g)) * u
                      [Moet "Qwen3.8": silu*up fused after the routed-expert GEMV;
                      Moet "MoE at decode": FC1 then FC2.]
  O7  FC2             o = W_d h
  O8  combine         y[t] = sum_i w_i o_i
                      [Tandem "How it works": nothing skipped or substituted.]
  O9  shared expert   y[t] += S(x_t), S = O6 + O7 with the shared expert's own
                      matrices, weight 1 for every token.  [DeepSeek V4 Flash article,
                      llama.cpp comparison: the GGUF file name marks a shared expert
                      ("SExpQ8"); the pages say nothing more, so this plain reading
                      (every token, weight 1, added after the routed combine) is R13.]
  O6' SwiGLU clamp    with a limit L > 0: g <- min(g, L), u <- clamp(u, -L, L)
                      before h = silu(g) * u.  [Moet "Quality vs native": the W2 path
                      had omitted the checkpoint's SwiGLU clamp.  The pages give
                      neither the form nor the constant: R14 takes the common form
                      (gate capped above, up clamped both ways) and leaves L a
                      parameter, 0 = off.  Parity unpinned: nothing on the pages fixes
                      a value to test the clamp against; the pins only check that it
                      leaves values inside [-L, L] alone and that this module and the
                      scalar brute force below agree.]
  O10 FP4 delta cache with a confidence gate
                      a routed pair (t, i) of expert e = S_i whose renormalised weight
                      w_i >= tau, and whose expert has a copy in the FP4 delta cache,
                      takes O6 and O7 with the copy's matrices (the expert in the
                      original FP4, MXFP4 here) instead of its 2-bit ones; every other
                      pair is unchanged, and so is its weight in O8.  [Moet "2-bit
                      experts on vLLM v0.24.0", first bullet: a delta cache and a
                      confidence gate bring FP4 back where it matters; "Benchmark
                      results", row glm-5.2-nvfp4: FP4 delta (auto) with a confidence
                      gate tau = 0.60.  The pages do not describe the mechanism: R15
                      reads the delta as the FP4 weights that replace the 2-bit ones
                      for a gated pair, R16 reads the gate's confidence as the pair's
                      renormalised routing weight; with tau >= 0.5 at most one pair
                      of a token (its first) can pass.]

Every value is computed in fp64 from the exact values of the stored fp16 / bf16 /
fp32 inputs.  Decoding is exact in fp64 (a product of two fp16 numbers).
"""
from __future__ import annotations

import itertools
import math
from fractions import Fraction
from typing import Dict, Optional, Sequence

import numpy as np

FMT_ABSENT = 0
FMT_VQ2 = 1
FMT_MXFP4 = 2

# ---------------------------------------------------------------------------------
# Reading stored values exactly
# ---------------------------------------------------------------------------------


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """Exact fp64 value of bf16 numbers given as u16 bit patterns (the top 16 bits
    of an IEEE binary32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f16_value(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.float16).astype(np.float64)


def x_value(x: np.ndarray, x_dtype: str) -> np.ndarray:
    """Exact fp64 value of activations stored as fp32 or as bf16 bits."""
    if x_dtype == "bf16":
        return bf16_value(x)
    if x_dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(x_dtype)


# ---------------------------------------------------------------------------------
# O1 / O1': decode
# ---------------------------------------------------------------------------------

def vq2_decode(codes: np.ndarray, scales: np.ndarray, codebook: np.ndarray) -> np.ndarray:
    """O1: decode one VQ2 matrix to fp64 [rows, in].

    R1 (sign bit): bit 7 of the word is the sign, bits 0..6 the codebook index.
    R2 (sign scope): the sign negates all four components of the codeword.
    R3 (vector axis): the four weights of a word are consecutive along the input
        (reduction) axis of one output row; codes are row-major [rows][in/4].
    R4 (scale group): one scale per 128 consecutive weights of a row.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    rows, n_words = codes.shape
    cb = f16_value(codebook)                                   # [128, 4]
    index = (codes & 0x7F).astype(np.int64)
    sign = np.where((codes & 0x80) != 0, -1.0, 1.0)
    vectors = cb[index] * sign[:, :, None]                     # [rows, in/4, 4]
    w = vectors.reshape(rows, n_words * 4)
    s = np.repeat(f16_value(scales), 128, axis=1)              # [rows, in]
    assert s.shape == w.shape, (s.shape, w.shape)
    return s * w


# OCP Microscaling Formats v1.0, FP4 (E2M1) element: 1 sign, 2 exponent, 1 mantissa
# bit, exponent bias 1, no inf/nan.  Magnitudes of codes 0..7:
E2M1_MAGNITUDE = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def e2m1_value(q: np.ndarray) -> np.ndarray:
    q = np.asarray(q, dtype=np.int64)
    mag = np.asarray(E2M1_MAGNITUDE, dtype=np.float64)[q & 7]
    return np.where((q & 8) != 0, -mag, mag)


def e8m0_value(e: np.ndarray) -> np.ndarray:
    """E8M0 shared scale 2^(e - 127); 255 encodes NaN."""
    e = np.asarray(e, dtype=np.int64)
    v = np.ldexp(1.0, e - 127)
    return np.where(e == 255, np.nan, v)


def mxfp4_decode(nibbles: np.ndarray, e8m0: np.ndarray) -> np.ndarray:
    """O1': decode one MXFP4 matrix to fp64 [rows, in].

    R5: blocks of 32 consecutive weights along the input axis; within a byte the
        low nibble holds the even-indexed weight.
    """
    nibbles = np.asarray(nibbles, dtype=np.uint8)
    rows, n_bytes = nibbles.shape
    q = np.empty((rows, n_bytes * 2), dtype=np.int64)
    q[:, 0::2] = nibbles & 0x0F
    q[:, 1::2] = nibbles >> 4
    scale = np.repeat(e8m0_value(e8m0), 32, axis=1)
    assert scale.shape == q.shape
    return e2m1_value(q) * scale


def decode_expert(expert: Dict[str, np.ndarray], codebook: np.ndarray):
    """(W_g [I,H], W_u [I,H], W_d [H,I]) of one expert in fp64."""
    fmt = int(expert["format"])
    if fmt == FMT_VQ2:
        return (vq2_decode(expert["codes_g"], expert["scales_g"], codebook),
                vq2_decode(expert["codes_u"], expert["scales_u"], codebook),
                vq2_decode(expert["codes_d"], expert["scales_d"], codebook))
    if fmt == FMT_MXFP4:
        return (mxfp4_decode(expert["nib_g"], expert["e8m0_g"]),
                mxfp4_decode(expert["nib_u"], expert["e8m0_u"]),
                mxfp4_decode(expert["nib_d"], expert["e8m0_d"]))
    raise ValueError(f"expert format {fmt} cannot be decoded")


# ---------------------------------------------------------------------------------
# O2..O5: routing
# ---------------------------------------------------------------------------------

def router_logits(router_w_bits: np.ndarray, x64: np.ndarray) -> np.ndarray:
    """O2: l[t, e] = sum_h W_r[e, h] x[t, h] (router weights stored as bf16)."""
    return np.asarray(x64, dtype=np.float64) @ bf16_value(router_w_bits).T


def softmax(logits: np.ndarray) -> np.ndarray:
    """O3, R6: a plain softmax over all experts (no bias, no group limit, no
    routed scaling factor)."""
    z = logits - logits.max(axis=-1, keepdims=True)
    ez = np.exp(z)
    return ez / ez.sum(axis=-1, keepdims=True)


def topk(logits: np.ndarray, k: int) -> np.ndarray:
    """O4, R7: per token, the k largest logits ordered by descending logit; equal
    logits are ordered by ascending expert id."""
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int64)
    for t in range(T):
        order = np.lexsort((np.arange(E), -logits[t]))   # primary -l, then id
        ids[t] = order[:k]
    return ids


def renormalise(p: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """O5, R8: w_i = p[S_i] / sum_{j in S} p[j] (applied after FC2, in O8)."""
    sel = np.take_along_axis(p, ids, axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


def route(router_w_bits: np.ndarray, x64: np.ndarray, k: int):
    logits = router_logits(router_w_bits, x64)
    p = softmax(logits)
    ids = topk(logits, k)
    return logits, ids, renormalise(p, ids)


# ---------------------------------------------------------------------------------
# O6..O8: experts and combine
# ---------------------------------------------------------------------------------

def silu(g: np.ndarray) -> np.ndarray:
    """R9: silu(g) = g * sigmoid(g) = g / (1 + exp(-g))."""
    return g / (1.0 + np.exp(-g))


def swiglu(g: np.ndarray, u: np.ndarray, limit: float = 0.0) -> np.ndarray:
    """O6 / O6': h = silu(g) * u; with limit L > 0 (R14), g is first capped at L and u
    clamped to [-L, L] (a NaN stays NaN)."""
    if limit > 0.0:
        g = np.where(g > limit, limit, g)
        u = np.where(u > limit, limit, np.where(u < -limit, -limit, u))
    return silu(g) * u


def expert_mlp(Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray, xs: np.ndarray,
               swiglu_limit: float = 0.0) -> Dict[str, np.ndarray]:
    """O6, O7 for tokens xs [m, H]: g, u, h [m, I] and o [m, H]."""
    g = xs @ Wg.T
    u = xs @ Wu.T
    h = swiglu(g, u, swiglu_limit)
    o = h @ Wd.T
    return {"g": g, "u": u, "h": h, "o": o}


def gate_passes(w: float, tau: Optional[float], has_copy: bool) -> bool:
    """O10 / R16: a pair uses its expert's FP4 copy when the expert has one and the
    pair's renormalised routing weight is at least tau."""
    return tau is not None and has_copy and w >= tau


def forward(layer, x64: np.ndarray, top_k: int,
            forced_selection: Optional[np.ndarray] = None, swiglu_limit: float = 0.0,
            shared: Optional[Dict[str, np.ndarray]] = None,
            fp4_copy=None, gate_tau: Optional[float] = None) -> Dict[str, np.ndarray]:
    """The whole routed-expert step for tokens x64 [T, H].

    ``layer`` provides ``codebook`` (fp16 [128,4]), ``router_w`` (bf16 bits
    [E,H]) and ``expert(e)`` (the storage arrays of expert e).
    ``forced_selection`` [T, k] replaces the top-k ids (used when a fp32 router
    picks a different but equally valid expert at a near-tie); the weights are
    then renormalised over the forced set.  ``swiglu_limit`` > 0 applies the clamp
    (O6') in every expert; ``shared`` (the storage arrays of a shared expert) adds
    O9.  ``fp4_copy(e)`` (the storage arrays of expert e's FP4 copy, or None) with
    ``gate_tau`` applies O10.

    Returns logits [T,E], ids [T,k], w [T,k], h [T,k,I], o [T,k,H], y [T,H],
    copy [T,k] (True where the pair took the FP4 copy), and with ``shared`` also
    h_shared [T,I], o_shared [T,H] (y includes o_shared).  Each expert (and each copy)
    is decoded once and applied to all of its tokens.
    """
    x64 = np.asarray(x64, dtype=np.float64)
    T, H = x64.shape
    logits = router_logits(layer.router_w, x64)
    p = softmax(logits)
    ids = topk(logits, top_k) if forced_selection is None else np.asarray(forced_selection, dtype=np.int64)
    w = renormalise(p, ids)
    copies = {}
    if fp4_copy is not None and gate_tau is not None:
        for e in sorted(set(ids.reshape(-1).tolist())):
            copies[e] = fp4_copy(e)
    use = np.array([[gate_passes(float(w[t, i]), gate_tau, copies.get(int(ids[t, i])) is not None)
                     for i in range(top_k)] for t in range(T)], dtype=bool).reshape(T, top_k)
    I = None
    h_all: Dict = {}
    o_all: Dict = {}
    for e, c in sorted(set((int(ids[t, i]), bool(use[t, i])) for t in range(T) for i in range(top_k))):
        pairs = [(t, i) for t in range(T) for i in range(top_k) if ids[t, i] == e and use[t, i] == c]
        tokens = [t for t, _ in pairs]
        Wg, Wu, Wd = decode_expert(copies[e] if c else layer.expert(e), layer.codebook)
        I = Wg.shape[0]
        r_ = expert_mlp(Wg, Wu, Wd, x64[tokens], swiglu_limit)
        for r, (t, i) in enumerate(pairs):
            h_all[(t, i)] = r_["h"][r]
            o_all[(t, i)] = r_["o"][r]
        del Wg, Wu, Wd
    h_out = np.zeros((T, top_k, I))
    o_out = np.zeros((T, top_k, H))
    y = np.zeros((T, H))
    for t in range(T):
        for i in range(top_k):
            h_out[t, i] = h_all[(t, i)]
            o_out[t, i] = o_all[(t, i)]
            y[t] += w[t, i] * o_all[(t, i)]
    out = {"logits": logits, "p": p, "ids": ids, "w": w, "h": h_out, "o": o_out, "y": y, "copy": use}
    if shared is not None:
        Wg, Wu, Wd = decode_expert(shared, layer.codebook)
        r_ = expert_mlp(Wg, Wu, Wd, x64, swiglu_limit)
        out["h_shared"], out["o_shared"] = r_["h"], r_["o"]
        y += r_["o"]
    return out


# ---------------------------------------------------------------------------------
# Brute force on tiny layers (pure Python scalars)
# ---------------------------------------------------------------------------------

def _scalar_weight(expert: Dict[str, np.ndarray], codebook: np.ndarray, mat: str, n: int, k: int) -> float:
    """One decoded weight, read straight from the storage arrays with Python scalars."""
    if int(expert["format"]) == FMT_VQ2:
        word = int(expert["codes_" + mat][n, k // 4])
        scale = float(expert["scales_" + mat][n, k // 128])
        comp = float(codebook[word & 0x7F, k % 4])
        return scale * (-comp if word >= 128 else comp)
    byte = int(expert["nib_" + mat][n, k // 2])
    q = (byte >> 4) if (k % 2) else (byte & 0xF)
    mag = E2M1_MAGNITUDE[q & 7]
    e = int(expert["e8m0_" + mat][n, k // 32])
    return math.ldexp(-mag if q & 8 else mag, e - 127)


def topk_bruteforce(logits_row: Sequence[float], k: int):
    """Enumerate every k-subset, keep the one with the largest exact logit sum;
    among equal sums the lexicographically smallest id tuple wins.  Returns the
    subset ordered by descending logit, ties by ascending id."""
    E = len(logits_row)
    exact = [Fraction(float(v)) for v in logits_row]
    best, best_sum = None, None
    for sub in itertools.combinations(range(E), k):
        s = sum(exact[e] for e in sub)
        if best is None or s > best_sum or (s == best_sum and sub < best):
            best, best_sum = sub, s
    return sorted(best, key=lambda e: (-exact[e], e))


def forward_bruteforce(layer, x64: np.ndarray, top_k: int, swiglu_limit: float = 0.0,
                       shared: Optional[Dict[str, np.ndarray]] = None,
                       fp4_copy=None, gate_tau: Optional[float] = None) -> np.ndarray:
    """y [T, H] from the dense all-expert form y[t] = sum_e M[t,e] * MLP_e(x_t) (+ the
    shared expert's MLP with weight 1), where M[t,e] is the renormalised routing weight
    for selected experts and 0 otherwise, and MLP_e uses expert e's FP4 copy where
    M[t,e] passes the gate (O10).  Scalar Python loops only; meant for the tiny layer."""
    x = [[float(v) for v in row] for row in np.asarray(x64, dtype=np.float64)]
    T, H = len(x), len(x[0])
    rw = bf16_value(layer.router_w)
    E = rw.shape[0]
    cb = f16_value(layer.codebook)
    Y = [[0.0] * H for _ in range(T)]
    for t in range(T):
        logits = []
        for e in range(E):
            acc = 0.0
            for j in range(H):
                acc += float(rw[e, j]) * x[t][j]
            logits.append(acc)
        m = max(logits)
        ex = [math.exp(v - m) for v in logits]
        total = sum(ex)
        p = [v / total for v in ex]
        sel = topk_bruteforce(logits, top_k)
        psel = sum(p[e] for e in sel)
        M = [p[e] / psel if e in sel else 0.0 for e in range(E)]
        mlps = []
        for e in range(E):
            cp = fp4_copy(e) if (fp4_copy is not None and gate_tau is not None and M[e] > 0.0) else None
            mlps.append((cp if (cp is not None and M[e] >= gate_tau) else layer.expert(e), M[e]))
        if shared is not None:
            mlps.append((shared, 1.0))
        for ex_arr, m_e in mlps:
            I = (ex_arr["codes_g"] if int(ex_arr["format"]) == FMT_VQ2 else ex_arr["nib_g"]).shape[0]
            h = []
            for n in range(I):
                g = sum(_scalar_weight(ex_arr, cb, "g", n, j) * x[t][j] for j in range(H))
                u = sum(_scalar_weight(ex_arr, cb, "u", n, j) * x[t][j] for j in range(H))
                if swiglu_limit > 0.0:
                    g = min(g, swiglu_limit)
                    u = max(-swiglu_limit, min(u, swiglu_limit))
                h.append(g / (1.0 + math.exp(-g)) * u)
            for n in range(H):
                o = sum(_scalar_weight(ex_arr, cb, "d", n, j) * h[j] for j in range(I))
                Y[t][n] += m_e * o
    return np.asarray(Y)


# ---------------------------------------------------------------------------------
# Encoder (nearest signed codeword) -- used to pin the decode by round trip
# ---------------------------------------------------------------------------------

def signed_codebook(codebook: np.ndarray) -> np.ndarray:
    """[256, 4] fp64: word b -> sgn(b) * CB[b & 0x7F]."""
    cb = f16_value(codebook)
    out = np.empty((256, 4))
    for b in range(256):
        out[b] = -cb[b & 0x7F] if b & 0x80 else cb[b & 0x7F]
    return out


def vq2_encode_nearest(w_over_s: np.ndarray, codebook: np.ndarray) -> np.ndarray:
    """Words [rows, in/4] whose signed codeword is nearest (squared distance) to each
    group of four values of w_over_s [rows, in]; ties go to the lowest word."""
    scb = signed_codebook(codebook)
    rows, n = w_over_s.shape
    v = w_over_s.reshape(rows, n // 4, 1, 4)
    d = ((v - scb[None, None, :, :]) ** 2).sum(axis=-1)        # [rows, in/4, 256]
    return np.argmin(d, axis=-1).astype(np.uint8)               # argmin: first minimum


# ---------------------------------------------------------------------------------
# Slot pool layout (read back from raw bytes)
# ---------------------------------------------------------------------------------

def _align256(n: int) -> int:
    return (n + 255) // 256 * 256


def slot_blocks(fmt: int, H: int, I: int):
    """Layout of one expert slot: list of (name, shape, dtype, byte offset) and total
    bytes.  Blocks in order gate, up, down payload then gate, up, down scales, each
    row-major and starting on a 256-byte boundary of the slot."""
    if fmt == FMT_VQ2:
        spec = [("codes_g", (I, H // 4), np.uint8), ("codes_u", (I, H // 4), np.uint8),
                ("codes_d", (H, I // 4), np.uint8), ("scales_g", (I, H // 128), np.float16),
                ("scales_u", (I, H // 128), np.float16), ("scales_d", (H, I // 128), np.float16)]
    elif fmt == FMT_MXFP4:
        spec = [("nib_g", (I, H // 2), np.uint8), ("nib_u", (I, H // 2), np.uint8),
                ("nib_d", (H, I // 2), np.uint8), ("e8m0_g", (I, H // 32), np.uint8),
                ("e8m0_u", (I, H // 32), np.uint8), ("e8m0_d", (H, I // 32), np.uint8)]
    else:
        raise ValueError(fmt)
    out, off = [], 0
    for name, shape, dt in spec:
        out.append((name, shape, dt, off))
        off = _align256(off + int(np.prod(shape)) * np.dtype(dt).itemsize)
    return out, off


def read_slot(pool: np.ndarray, byte_offset: int, fmt: int, H: int, I: int) -> Dict[str, np.ndarray]:
    blocks, _ = slot_blocks(fmt, H, I)
    out: Dict[str, np.ndarray] = {"format": np.int32(fmt)}
    for name, shape, dt, off in blocks:
        nbytes = int(np.prod(shape)) * np.dtype(dt).itemsize
        raw = pool[byte_offset + off: byte_offset + off + nbytes]
        out[name] = np.frombuffer(raw.tobytes(), dtype=dt).reshape(shape)
    return out


# ---------------------------------------------------------------------------------
# fp32 dot-product error bound (accepting near-tie selections)
# ---------------------------------------------------------------------------------

def fp32_dot_error_bound(router_w_bits: np.ndarray, x64: np.ndarray) -> np.ndarray:
    """delta[t, e] = gamma_H * sum_h |W_r[e,h] x[t,h]|, gamma_H = H u / (1 - H u),
    u = 2^-24: a bound on |fp32 dot - exact dot| for any summation order with exact
    products (bf16 x bf16 and bf16 x fp32-from-bf16 products are exact in fp32).
    For fp32 activations the products round once more, which adds u per term; the
    bound below uses (H + 1) to cover it."""
    x64 = np.asarray(x64, dtype=np.float64)
    H = x64.shape[1]
    u = 2.0 ** -24
    n = H + 1
    gamma = n * u / (1 - n * u)
    return gamma * (np.abs(x64) @ np.abs(bf16_value(router_w_bits)).T)


def selection_is_valid(gpu_ids: np.ndarray, logits: np.ndarray, delta: np.ndarray, k: int) -> bool:
    """True when gpu_ids [T,k] is a correct top-k for some logits within delta of the
    fp64 logits: every chosen expert must not be beaten by an unchosen one by more
    than the two error bounds, the ids in a row are distinct, and the order is
    descending up to the same tolerance."""
    T, E = logits.shape
    for t in range(T):
        row = [int(v) for v in gpu_ids[t]]
        if len(set(row)) != k or min(row) < 0 or max(row) >= E:
            return False
        chosen = set(row)
        for a in row:
            for b in range(E):
                if b in chosen:
                    continue
                if logits[t, b] - logits[t, a] > delta[t, a] + delta[t, b]:
                    return False
        for i in range(k - 1):
            a, b = row[i], row[i + 1]
            if logits[t, b] - logits[t, a] > delta[t, a] + delta[t, b]:
                return False
    return True
