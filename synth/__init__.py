"""Seeded synthetic workloads for the LRMoE backward hot path (input generation only).

This module builds the inputs that both the GPU library and the CPU oracle are fed: routing
indices and gate weights from a biased random router, MoE-output gradients ``g``, saved SwiGLU
activations ``phi`` in the forward dispatch layout, and FC2 weights ``W``; for the rest of the
expert backward also the saved FC1 outputs (gate and up halves), the layer input ``x`` and the FC1
weights ``W1``.  It holds none of the
method's arithmetic (no counting, quotas, scores, selection, compaction or gradients); the router
below is the forward gating step that precedes the method, reproduced only to obtain realistic
routing skew.

Workload shapes follow the LRMoE paper's evaluation models (Sec. 4.1: Qwen3-30B-A3B with 128
experts, top-8, H=2048, F=768, 32768 tokens per GPU) and the GLM-4.5-Air shape listed in the
TopoEP paper's model table (hidden 4096, expert intermediate 1408).  The router follows the
TopoEP paper's synthetic-routing recipe (Sec. 6, skew experiments: random router logits plus a
constant offset per expert), here with Zipf-shaped per-expert offsets.

Random values come from the counter-based SplitMix64 + Box-Muller generator in ``rng.c``; every
value depends only on its identity (seed, stream, index), never on the array layout.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_LIB = None

# Stream ids of the counter-based generator.
S_X, S_WR, S_G, S_A, S_C, S_W, S_GSCALE, S_PHISCALE, S_TIES, S_KEYS, S_W1 = range(1, 12)

_KIND = {"f64": 0, "f32": 1, "bf16": 2}


def build(force: bool = False) -> str:
    """Compile ``rng.c`` into ``libsynth.so`` (gcc, OpenMP)."""
    global _LIB
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp,
                               os.path.join(_HERE, "rng.c"), "-lm"])
        os.replace(tmp, _SO)
        _LIB = None
    return _SO


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        u64, i64, vp, dbl = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
        lib.synth_stream_key.argtypes = [u64, u64]
        lib.synth_stream_key.restype = u64
        lib.synth_normals.argtypes = [u64, u64, i64, i64, vp]
        lib.synth_uniforms_f32.argtypes = [u64, u64, i64, i64, vp]
        lib.synth_rows.argtypes = [u64, u64, vp, i64, i64, i64, dbl, dbl, u64, ctypes.c_int, vp]
        lib.synth_swiglu_rows.argtypes = [u64, u64, u64, vp, i64, i64, dbl, u64, ctypes.c_int, vp]
        lib.synth_swiglu_context.argtypes = [u64, u64, u64, vp, i64, i64, dbl, u64, ctypes.c_int,
                                             vp]
        _LIB = lib
    return _LIB


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def normals(seed: int, stream: int, start: int, n: int) -> np.ndarray:
    out = np.empty(n, np.float64)
    _lib().synth_normals(seed, stream, start, n, _ptr(out))
    return out


def uniforms_f32(seed: int, stream: int, start: int, n: int) -> np.ndarray:
    out = np.empty(n, np.float32)
    _lib().synth_uniforms_f32(seed, stream, start, n, _ptr(out))
    return out


def pair_keys(sp: "Spec") -> np.ndarray:
    """One uniform key per pair p in [0, T*k), float32: the random draws of a random-drop
    selection, generated here and handed to both sides."""
    return uniforms_f32(sp.seed, S_KEYS, 0, sp.T * sp.k)


def rows(seed, stream, nrows, ncols, *, scale=1.0, src_row=None, row0=0, row_sigma=0.0,
         row_stream=0, kind="f32") -> np.ndarray:
    dt = {"f64": np.float64, "f32": np.float32, "bf16": np.uint16}[kind]
    out = np.empty((nrows, ncols), dt)
    src = None if src_row is None else np.ascontiguousarray(src_row, np.int64)
    _lib().synth_rows(seed, stream, _ptr(src), row0, nrows, ncols, scale, row_sigma, row_stream,
                      _KIND[kind], _ptr(out))
    return out


def swiglu_rows(seed, src_pair, ncols, *, row_sigma=0.0, kind="bf16") -> np.ndarray:
    dt = {"f64": np.float64, "f32": np.float32, "bf16": np.uint16}[kind]
    src = np.ascontiguousarray(src_pair, np.int64)
    out = np.empty((src.shape[0], ncols), dt)
    _lib().synth_swiglu_rows(seed, S_A, S_C, _ptr(src), src.shape[0], ncols, row_sigma,
                             S_PHISCALE, _KIND[kind], _ptr(out))
    return out


def swiglu_context_rows(seed, src_pair, ncols, *, row_sigma=0.0, kind="bf16") -> np.ndarray:
    """[rows, 2*ncols]: the gate pre-activation a, then the (row-scaled) up projection c, of the
    draws that swiglu_rows combines into phi."""
    dt = {"f64": np.float64, "f32": np.float32, "bf16": np.uint16}[kind]
    src = np.ascontiguousarray(src_pair, np.int64)
    out = np.empty((src.shape[0], 2 * ncols), dt)
    _lib().synth_swiglu_context(seed, S_A, S_C, _ptr(src), src.shape[0], ncols, row_sigma,
                                S_PHISCALE, _KIND[kind], _ptr(out))
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 values (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------------------------
# Workload definitions
# --------------------------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Spec:
    """Shape, router and quota recipe of one synthetic workload."""
    name: str
    T: int
    k: int
    E: int
    e_lo: int
    E_loc: int
    h: int
    d: int
    dtype: str                 # "f32" or "bf16": element type of g, phi, W
    zipf_s: float
    rho_num: int
    rho_den: int
    cap_abs: int = -1          # absolute per-expert quota cap, -1 = none
    g_row_sigma: float = 0.0   # LogNormal(0, sigma) scale of each g row
    phi_row_sigma: float = 0.0  # LogNormal(0, sigma) scale of each phi row
    skew_hot0: bool = False    # expert 0 forced to ~30 % of local pairs, 3 locals forced empty
    dup_frac: float = 0.0      # fraction of tokens that duplicate another token
    seed: int = 1000


SPECS = {
    # Tiny fp32 layer: E=8, top-2, all experts local, q = min(n, floor(0.6*T*k/E)).
    0: Spec("tiny-fp32 E8 top2 T4096 h256 d512", 4096, 2, 8, 0, 8, 256, 512, "f32", 1.0, 3, 5,
            seed=1000),
    # Qwen3-30B-A3B shape, one GPU's share (16 of 128 experts), rho = 0.5.
    1: Spec("qwen3-30b-a3b share E128/16 top8 T32768 h2048 d768", 32768, 8, 128, 0, 16, 2048, 768,
            "bf16", 1.2, 1, 2, seed=1001),
    # GLM4.5-106B-A12B shape, one GPU's share, g rows scaled by LogNormal(0, 1).
    2: Spec("glm4.5-106b-a12b share E128/16 top8 T32768 h4096 d1408", 32768, 8, 128, 0, 16, 4096,
            1408, "bf16", 1.2, 1, 2, g_row_sigma=1.0, seed=1002),
    # Extreme skew on the Qwen3 shape; phi rows scaled by LogNormal(0, 1.5).
    3: Spec("qwen3 extreme-skew share E128/16 top8 T32768 h2048 d768", 32768, 8, 128, 0, 16, 2048,
            768, "bf16", 1.5, 1, 2, phi_row_sigma=1.5, skew_hot0=True, seed=1003),
    # Whole layer on one GPU (128 local experts), rho = 0.4, cap 1.25*T*k/E, 1 % duplicated tokens.
    4: Spec("qwen3 whole-layer E128/128 top8 T16384 h2048 d768", 16384, 8, 128, 0, 128, 2048, 768,
            "bf16", 1.2, 2, 5, cap_abs=(5 * 16384 * 8) // (4 * 128), dup_frac=0.01, seed=1004),
    # DeepSeek-V2 expert shape (160 experts, top-6, hidden 5120, expert FFN 1536), one GPU's share
    # of an 8-way expert-parallel layer (20 local experts), rho = 0.5.
    5: Spec("deepseek-v2 share E160/20 top6 T16384 h5120 d1536", 16384, 6, 160, 0, 20, 5120, 1536,
            "bf16", 1.2, 1, 2, seed=1005),
}

# The retention sweep of the extreme-skew workload.
RHO_SWEEP_3 = [(1, 1), (3, 4), (1, 2), (1, 4)]


def spec(cfg: int, **overrides) -> Spec:
    """The spec of workload ``cfg`` with optional field overrides (e.g. a smaller T)."""
    s = SPECS[cfg]
    if overrides:
        s = dataclasses.replace(s, **overrides)
        if "cap_abs" not in overrides and cfg == 4:
            s = dataclasses.replace(s, cap_abs=(5 * s.T * s.k) // (4 * s.E))
    return s


@dataclasses.dataclass
class Workload:
    spec: Spec
    topk_idx: np.ndarray   # int32 [T*k], pair p = t*k + j, slot j in descending-logit order
    topk_w: np.ndarray     # float32 [T*k], routing weight alpha of pair p
    g: np.ndarray          # [T, h] float32 or bf16 bits (uint16)
    phi: np.ndarray        # [L, d] rows in forward dispatch layout (expert-major, p ascending)
    W: np.ndarray          # [E_loc, h, d] FC2 weights of the local experts
    layout_pairs: np.ndarray  # int64 [L] the pair of each phi row (the layout convention)
    router_bias: np.ndarray   # float64 [E]
    dup_src: np.ndarray       # int64 [T] source token of every token (itself unless duplicated)

    @property
    def L(self) -> int:
        return int(self.layout_pairs.shape[0])


def _zipf_bias(ranks: np.ndarray, s: float) -> np.ndarray:
    w = ranks.astype(np.float64) ** (-s)
    return 1.5 * np.log(w / w.sum())


def _router_bias_plain(sp: Spec) -> np.ndarray:
    # Expert e has Zipf rank e+1: expert 0 is the hottest.
    return _zipf_bias(np.arange(1, sp.E + 1), sp.zipf_s)


def _router_bias_skew_base(sp: Spec) -> np.ndarray:
    """Extreme-skew bias for experts 1..E-1 (expert 0 is set by bisection later).

    Local experts 1..E_loc-1 take every 4th Zipf rank (1, 5, 9, ...), non-local experts fill the
    remaining ranks in id order; the last three local experts are never routed to (bias -inf).
    """
    E = sp.E
    rank = np.zeros(E, np.int64)
    local_ranks = [1 + 4 * (e - 1) for e in range(1, sp.E_loc)]
    for e, r in zip(range(1, sp.E_loc), local_ranks):
        rank[e] = r
    free = [r for r in range(1, E) if r not in set(local_ranks)]
    for e, r in zip(range(sp.E_loc, E), free):
        rank[e] = r
    b = np.zeros(E)
    b[1:] = _zipf_bias(rank[1:], sp.zipf_s)
    b[sp.E_loc - 3:sp.E_loc] = -np.inf
    return b


def _base_logits(sp: Spec, src_tok: np.ndarray) -> np.ndarray:
    """x . W_r in fp64 from fp32-rounded x ~ N(0,1) and W_r ~ N(0, 1/h)."""
    Wr = rows(sp.seed, S_WR, sp.h, sp.E, scale=1.0 / np.sqrt(sp.h), kind="f32").astype(np.float64)
    out = np.empty((sp.T, sp.E), np.float64)
    CH = 4096
    for t0 in range(0, sp.T, CH):
        t1 = min(sp.T, t0 + CH)
        x = rows(sp.seed, S_X, t1 - t0, sp.h, src_row=src_tok[t0:t1], kind="f32")
        out[t0:t1] = x.astype(np.float64) @ Wr
    return out


def _bisect_hot0(sp: Spec, logits_wo0: np.ndarray, base0: np.ndarray) -> float:
    """Bias of expert 0 such that it receives 29.5-30.5 % of the local pairs (60-step bisection)."""
    k, E_loc, e_lo = sp.k, sp.E_loc, sp.e_lo
    others = logits_wo0[:, 1:]
    order = np.argsort(-others, axis=1, kind="stable")[:, :k]      # top-k among experts 1..E-1
    top_ids = order + 1
    kth = np.take_along_axis(others, order[:, k - 1:k], axis=1)[:, 0]
    is_local = (top_ids >= e_lo) & (top_ids < e_lo + E_loc)
    loc_cnt = is_local.sum(axis=1)
    kth_local = is_local[:, k - 1]

    def frac(b0):
        inn = (base0 + b0) >= kth            # expert 0 wins ties (lowest id)
        n0 = int(inn.sum())
        L = int(loc_cnt.sum() - (inn & kth_local).sum()) + n0
        return n0 / max(L, 1)

    lo, hi = -30.0, 30.0
    b = 0.0
    for _ in range(60):
        b = 0.5 * (lo + hi)
        f = frac(b)
        if 0.295 <= f <= 0.305:
            break
        if f < 0.30:
            lo = b
        else:
            hi = b
    return b


def _route(logits: np.ndarray, k: int):
    order = np.argsort(-logits, axis=1, kind="stable")[:, :k]        # ties -> lower expert id
    top = np.take_along_axis(logits, order, axis=1)
    m = top[:, :1]
    w = np.exp(top - m)
    alpha = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    return order.astype(np.int32), alpha


def make(cfg, **overrides) -> Workload:
    """Generate workload ``cfg`` (an int id or a Spec) with optional Spec overrides."""
    sp = cfg if isinstance(cfg, Spec) else spec(cfg, **overrides)
    T, k = sp.T, sp.k

    # Duplicated tokens (exact ties): copies take x, g and phi of a seeded source token.
    src_tok = np.arange(T, dtype=np.int64)
    n_dup = int(round(sp.dup_frac * T))
    if n_dup > 0:
        perm = np.argsort(normals(sp.seed, S_TIES, 0, T), kind="stable")
        copies, sources = perm[:n_dup], perm[n_dup:2 * n_dup]
        src_tok[copies] = sources

    logits = _base_logits(sp, src_tok)
    if sp.skew_hot0:
        bias = _router_bias_skew_base(sp)
        base0 = logits[:, 0].copy()
        with np.errstate(invalid="ignore"):
            lw = logits + bias
        b0 = _bisect_hot0(sp, lw, base0)
        bias[0] = b0
    else:
        bias = _router_bias_plain(sp)
    logits = logits + bias
    topk_idx, alpha = _route(logits, k)
    del logits

    idx = topk_idx.reshape(-1)
    p_all = np.arange(T * k, dtype=np.int64)
    loc = (idx >= sp.e_lo) & (idx < sp.e_lo + sp.E_loc)
    lp = p_all[loc]
    layout_pairs = lp[np.argsort(idx[loc], kind="stable")]        # expert-major, p ascending

    g = rows(sp.seed, S_G, T, sp.h, src_row=src_tok, row_sigma=sp.g_row_sigma,
             row_stream=S_GSCALE, kind=sp.dtype)
    src_pair = src_tok[layout_pairs // k] * k + layout_pairs % k
    phi = swiglu_rows(sp.seed, src_pair, sp.d, row_sigma=sp.phi_row_sigma, kind=sp.dtype)
    W = rows(sp.seed, S_W, sp.E_loc * sp.h, sp.d, row0=sp.e_lo * sp.h,
             scale=1.0 / np.sqrt(sp.d), kind=sp.dtype).reshape(sp.E_loc, sp.h, sp.d)
    return Workload(sp, idx.astype(np.int32).copy(), alpha.reshape(-1).copy(), g, phi, W,
                    layout_pairs, bias, src_tok)


@dataclasses.dataclass
class LayerInputs:
    """Inputs of the rest of the expert backward (FC1 and the activation) of a workload."""
    ac: np.ndarray   # [L, 2d] saved FC1 outputs per forward row: gate pre-activation a | up c
    x: np.ndarray    # [T, h] the layer input of every token (FC1's input)
    W1: np.ndarray   # [E_loc, 2d, h] FC1 weights of the local experts: gate rows, then up rows


def layer_inputs(w: Workload) -> LayerInputs:
    """Saved FC1 outputs, token inputs and FC1 weights for workload ``w``.

    a and c are the draws behind phi (phi = SiLU(a) * c, row scale folded into c), x is the router
    input of every token rounded to the storage type, W1 ~ N(0, 1/h).  Duplicated tokens copy their
    source's x and context like every other per-token value."""
    sp = w.spec
    src_pair = w.dup_src[w.layout_pairs // sp.k] * sp.k + w.layout_pairs % sp.k
    ac = swiglu_context_rows(sp.seed, src_pair, sp.d, row_sigma=sp.phi_row_sigma, kind=sp.dtype)
    x = rows(sp.seed, S_X, sp.T, sp.h, src_row=w.dup_src, kind=sp.dtype)
    W1 = rows(sp.seed, S_W1, sp.E_loc * 2 * sp.d, sp.h, row0=sp.e_lo * 2 * sp.d,
              scale=1.0 / np.sqrt(sp.h), kind=sp.dtype).reshape(sp.E_loc, 2 * sp.d, sp.h)
    return LayerInputs(ac, x, W1)


def policy(sp: Spec, *, full: bool = False, rho=None, kind: str = "cap", cap=None) -> dict:
    """Quota policy of a workload (its retention fraction and cap unless overridden); `kind`
    names the split ("cap", "proportional" or "waterfill")."""
    num, den = (sp.rho_num, sp.rho_den) if rho is None else rho
    c = sp.cap_abs if cap is None else cap
    return {"full": int(full), "rho_num": int(num), "rho_den": int(den), "cap_abs": int(c),
            "kind": kind}
