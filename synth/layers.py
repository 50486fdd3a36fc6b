"""Seeded generators for synthetic layers, predictors and tokens.

Every tensor is a stack of 1024-row blocks; block ``k`` of tensor ``t`` of layer
``l`` in configuration ``c`` is drawn from
``Generator(PCG64(SeedSequence(seed, spawn_key=(c, l, t, k))))``.  Any block of
any layer can therefore be regenerated alone, on any host, bit-identically, and
blocks can be drawn in parallel threads (numpy releases the GIL while it fills
large arrays).

Statistics follow the PowerInfer pages: neuron firing follows a power law
(project page, "Core technical principle": a few hot neurons fire on most
inputs, cold ones depend on the input; paper summary, "Key Results": 26 % of
neurons carry 80 % of the activations) at the sparsity the pages quote (about
90 %, project page "Supported models").  Nothing here evaluates the FFN.
"""

from __future__ import annotations

import functools
import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional

import numpy as np
from scipy.special import ndtri

from .configs import LayerConfig

BLOCK_ROWS = 1024
P_CAP = 0.99

T_PERM, T_WGATE, T_WUP, T_WDOWN, T_P1, T_P2, T_X = range(7)

_NP_DTYPE = {"f32": np.float32, "f16": np.float16}


def _rng(seed: int, key: tuple) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


def _threads() -> int:
    env = os.environ.get("PI_SYNTH_THREADS")
    if env:
        return max(1, int(env))
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_block(seed: int, key: tuple, rows: int, cols: int, scale: float) -> np.ndarray:
    """One block of N(0, scale^2) float32 values, shape [rows][cols]."""
    a = _rng(seed, key).standard_normal((rows, cols), dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return a


def normal_matrix(seed: int, key: tuple, rows: int, cols: int, scale: float,
                  row_start: int = 0, row_stop: Optional[int] = None,
                  out_dtype=np.float32, pool: Optional[ThreadPoolExecutor] = None) -> np.ndarray:
    """Rows [row_start, row_stop) of a blocked N(0, scale^2) matrix, cast to out_dtype."""
    row_stop = rows if row_stop is None else row_stop
    out = np.empty((row_stop - row_start, cols), dtype=out_dtype)
    b0, b1 = row_start // BLOCK_ROWS, (row_stop - 1) // BLOCK_ROWS if row_stop > row_start else -1

    def fill(b: int) -> None:
        r0 = b * BLOCK_ROWS
        r1 = min(rows, r0 + BLOCK_ROWS)
        blk = normal_block(seed, key + (b,), r1 - r0, cols, scale)
        lo, hi = max(r0, row_start), min(r1, row_stop)
        out[lo - row_start:hi - row_start] = blk[lo - r0:hi - r0].astype(out_dtype)

    blocks = list(range(b0, b1 + 1))
    if pool is not None and len(blocks) > 1:
        list(pool.map(fill, blocks))
    else:
        for b in blocks:
            fill(b)
    return out


# ----------------------------------------------------------------------------
# Firing probabilities
# ----------------------------------------------------------------------------

def _zipf_base(n: int, s: float) -> np.ndarray:
    return np.arange(1, n + 1, dtype=np.float64) ** (-s)


def _scale_for_density(base: np.ndarray, density: float, cap: float) -> float:
    """Bisection on c so that mean(min(cap, c k^-s)) == density."""
    if not (0.0 < density < cap):
        raise ValueError("density must lie in (0, cap)")
    lo, hi = 0.0, 1.0
    while np.minimum(cap, hi * base).mean() < density:
        hi *= 2.0
    for _ in range(100):
        mid = 0.5 * (lo + hi)
        if np.minimum(cap, mid * base).mean() < density:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def firing_probs_by_rank(n: int, density: float, s: float, cap: float = P_CAP) -> np.ndarray:
    """Descending power-law firing probabilities p_k = min(cap, c k^-s), mean = density."""
    base = _zipf_base(n, s)
    return np.minimum(cap, _scale_for_density(base, density, cap) * base)


def top_share(p_desc: np.ndarray, frac: float) -> float:
    k = int(math.ceil(frac * p_desc.size))
    return float(p_desc[:k].sum() / p_desc.sum())


@functools.lru_cache(maxsize=None)
def solve_zipf_exponent(n: int, density: float, frac: float, share: float,
                        cap: float = P_CAP) -> float:
    """Exponent s for which the top `frac` of neurons carry `share` of the firing mass."""
    lo, hi = 0.3, 4.0
    for _ in range(60):
        mid = 0.5 * (lo + hi)
        if top_share(firing_probs_by_rank(n, density, mid, cap), frac) < share:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def zipf_exponent(cfg: LayerConfig) -> float:
    if cfg.zipf_s is not None:
        return cfg.zipf_s
    frac, share = cfg.top_share
    return solve_zipf_exponent(cfg.d_ffn, cfg.density, frac, share)


def firing_probs(cfg: LayerConfig, layer: int, seed: int = 0) -> np.ndarray:
    """Per-neuron firing probability: power law by rank, ranks dealt to neurons by a seeded permutation."""
    p_rank = firing_probs_by_rank(cfg.d_ffn, cfg.density, zipf_exponent(cfg))
    perm = _rng(seed, (cfg.cfg_id, layer, T_PERM)).permutation(cfg.d_ffn)
    p = np.empty(cfg.d_ffn, dtype=np.float64)
    p[perm] = p_rank
    return p


# ----------------------------------------------------------------------------
# int4 group-32 encoding (data encoding only; decoding lives in the consumers)
# ----------------------------------------------------------------------------

def pack_nibbles(q: np.ndarray) -> np.ndarray:
    """int values in [-8, 7], shape [rows][cols] (cols even) -> uint8 [rows][cols/2].

    Element 2j goes to the low nibble of byte j, element 2j+1 to the high nibble,
    both as 4-bit two's complement.
    """
    q = np.asarray(q)
    if q.shape[-1] % 2:
        raise ValueError("column count must be even")
    if q.min(initial=0) < -8 or q.max(initial=0) > 7:
        raise ValueError("int4 values must lie in [-8, 7]")
    u = (q.astype(np.int16) & 0xF).astype(np.uint8)
    return (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)


def quantize_q4g32(w: np.ndarray):
    """Symmetric int4 with one fp16 scale per 32 consecutive elements of a row.

    s = fp16(max|w| / 7); q = clamp(round_half_even(w / s), -8, 7); s == 0 gives q = 0.
    Returns (packed uint8 [rows][cols/2], scales fp16 [rows][cols/32]).
    """
    rows, cols = w.shape
    if cols % 32:
        raise ValueError("column count must be a multiple of 32")
    g = w.reshape(rows, cols // 32, 32).astype(np.float64)
    s16 = (np.abs(g).max(axis=2) / 7.0).astype(np.float16)
    s = s16.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s > 0, np.rint(g / np.where(s > 0, s, 1.0)), 0.0)
    q = np.clip(q, -8, 7).astype(np.int8).reshape(rows, cols)
    return pack_nibbles(q), s16


# ----------------------------------------------------------------------------
# Layers
# ----------------------------------------------------------------------------

@dataclass
class Layer:
    """One FFN layer's tensors, all neuron-major ([n][...]).

    w_gate / w_up / w_down_t: [n][d] in f32/f16, or uint8 [n][d/2] packed int4
    (then s_* hold fp16 [n][d/32] scales).  w_down_t row i is neuron i's
    down-projection weights.  b: float32 [n] bias on the gate (gated) or on the
    up projection (non-gated).  p1 [r][d], p2 [n][r], b_p float32 [n].
    """

    d_model: int
    d_ffn: int
    rank: int
    gated: bool
    w_dtype: str
    p_dtype: str
    act_dtype: str
    tau: float
    w_gate: Optional[np.ndarray]
    w_up: np.ndarray
    w_down_t: np.ndarray
    s_gate: Optional[np.ndarray]
    s_up: Optional[np.ndarray]
    s_down: Optional[np.ndarray]
    b: np.ndarray
    p1: Optional[np.ndarray]
    p2: Optional[np.ndarray]
    b_p: Optional[np.ndarray]
    p: Optional[np.ndarray] = None      # firing probabilities used to place the biases
    name: str = ""
    index: int = 0


def _weight(seed, key, n, d, w_dtype, pool):
    """Returns (stored, scales, row_norms_of_source_or_stored)."""
    if w_dtype == "q4g32":
        src = normal_matrix(seed, key, n, d, 1.0 / math.sqrt(d), pool=pool)
        norms = np.sqrt(np.einsum("ij,ij->i", src.astype(np.float64), src.astype(np.float64)))
        q, s = quantize_q4g32(src)
        return q, s, norms
    dt = _NP_DTYPE[w_dtype]
    w = normal_matrix(seed, key, n, d, 1.0 / math.sqrt(d), out_dtype=dt, pool=pool)
    w64 = w.astype(np.float64)
    norms = np.sqrt(np.einsum("ij,ij->i", w64, w64))
    return w, None, norms


def make_layer(cfg: LayerConfig, layer: int, seed: int = 0, with_predictor: bool = True,
               threads: Optional[int] = None) -> Layer:
    """Regenerate layer `layer` of configuration `cfg` bit-identically."""
    d, n, r = cfg.d_model, cfg.d_ffn, cfg.rank
    p = firing_probs(cfg, layer, seed)
    nthreads = threads or _threads()
    with ThreadPoolExecutor(nthreads) as pool:
        w_gate = s_gate = None
        if cfg.gated:
            w_gate, s_gate, gate_norms = _weight(seed, (cfg.cfg_id, layer, T_WGATE), n, d, cfg.w_dtype, pool)
        w_up, s_up, up_norms = _weight(seed, (cfg.cfg_id, layer, T_WUP), n, d, cfg.w_dtype, pool)
        w_down_t, s_down, _ = _weight(seed, (cfg.cfg_id, layer, T_WDOWN), n, d, cfg.w_dtype, pool)
        # Bias: g_i = x . w_i + b_i with x ~ N(0, I) is N(b_i, |w_i|^2), so
        # b_i = |w_i| * Phi^-1(p_i) makes P(g_i > 0) = p_i.
        sigma = gate_norms if cfg.gated else up_norms
        b = (sigma * ndtri(p)).astype(np.float32)

        p1 = p2 = b_p = None
        if with_predictor and r > 0:
            pdt = _NP_DTYPE[cfg.p_dtype]
            p1 = normal_matrix(seed, (cfg.cfg_id, layer, T_P1), r, d, 1.0 / math.sqrt(d), out_dtype=pdt, pool=pool)
            p2 = normal_matrix(seed, (cfg.cfg_id, layer, T_P2), n, r, 1.0 / math.sqrt(r), out_dtype=pdt, pool=pool)
            b_p = predictor_bias(p1, p2, p)
    return Layer(d_model=d, d_ffn=n, rank=r if with_predictor else 0, gated=cfg.gated,
                 w_dtype=cfg.w_dtype, p_dtype=cfg.p_dtype, act_dtype=cfg.act_dtype, tau=cfg.tau,
                 w_gate=w_gate, w_up=w_up, w_down_t=w_down_t, s_gate=s_gate, s_up=s_up, s_down=s_down,
                 b=b, p1=p1, p2=p2, b_p=b_p, p=p, name=cfg.name, index=layer)


def predictor_bias(p1: np.ndarray, p2: np.ndarray, p: np.ndarray) -> np.ndarray:
    """Output bias that places the predictor's firing rate at p_i.

    Hidden unit j is max(N(0, |P1_j|^2), 0) for x ~ N(0, I): mean |P1_j|/sqrt(2 pi),
    variance |P1_j|^2 (1/2 - 1/(2 pi)).  Treating hidden units as independent,
    the logit is roughly N(mu_i + b_i, s_i^2), so b_i = -mu_i + s_i Phi^-1(p_i).
    """
    p1n = np.sqrt(np.einsum("ij,ij->i", p1.astype(np.float64), p1.astype(np.float64)))
    p2d = p2.astype(np.float64)
    mu = (p2d @ p1n) / math.sqrt(2.0 * math.pi)
    var = (p2d * p2d) @ (p1n * p1n) * (0.5 - 1.0 / (2.0 * math.pi))
    return (-mu + np.sqrt(var) * ndtri(p)).astype(np.float32)


def make_tokens(cfg: LayerConfig, layer: int, count: int, start: int = 0, seed: int = 0) -> np.ndarray:
    """Token inputs x ~ N(0, I) for layer `layer`, rows [start, start+count), in the act dtype."""
    if start < 0 or start + count > cfg.tokens:
        raise ValueError(f"tokens [{start}, {start + count}) outside [0, {cfg.tokens})")
    return normal_matrix(seed, (cfg.cfg_id, layer, T_X), cfg.tokens, cfg.d_model, 1.0,
                         row_start=start, row_stop=start + count, out_dtype=_NP_DTYPE[cfg.act_dtype])


# ----------------------------------------------------------------------------
# Integer-lattice layers: every sum the method forms is an exact small integer
# (or a dyadic rational for int4), so any summation order gives the same value.
# ----------------------------------------------------------------------------

def _ternary(rng, shape, p_nonzero):
    v = rng.integers(-1, 2, size=shape)
    keep = rng.random(shape) < p_nonzero
    return np.where(keep, v, 0)


def make_lattice_layer(d: int, n: int, r: int, gated: bool, w_dtype: str = "f16",
                       p_dtype: str = "f16", act_dtype: str = "f16", seed: int = 1,
                       w_nonzero: float = 0.25, down_nonzero: float = 1 / 32,
                       tau: float = 0.5) -> Layer:
    """Small-integer layer: weights in {-1,0,1} (int4: q in [-8,7] with power-of-two scales),
    integer biases.  Exact in fp16/fp32 storage."""
    rng = _rng(seed, (99, d, n, r, int(gated)))
    wnz = min(1.0, w_nonzero * 64.0 / d) if d > 64 else w_nonzero

    def wmat(nonzero):
        if w_dtype == "q4g32":
            q = _ternary(rng, (n, d), nonzero) * rng.integers(1, 8, size=(n, d))
            q = np.clip(q, -8, 7)
            scales = np.float16(2.0) ** rng.integers(-1, 2, size=(n, d // 32)).astype(np.float16)
            return pack_nibbles(q), scales.astype(np.float16)
        return _ternary(rng, (n, d), nonzero).astype(_NP_DTYPE[w_dtype]), None

    w_gate = s_gate = None
    if gated:
        w_gate, s_gate = wmat(wnz)
    w_up, s_up = wmat(wnz)
    w_down_t, s_down = wmat(down_nonzero)
    b = rng.integers(-2, 3, size=n).astype(np.float32)
    p1 = p2 = b_p = None
    if r > 0:
        pdt = _NP_DTYPE[p_dtype]
        p1 = _ternary(rng, (r, d), min(1.0, 16.0 / d)).astype(pdt)
        p2 = _ternary(rng, (n, r), min(1.0, 8.0 / r)).astype(pdt)
        b_p = rng.integers(-2, 2, size=n).astype(np.float32)
    return Layer(d_model=d, d_ffn=n, rank=r, gated=gated, w_dtype=w_dtype, p_dtype=p_dtype,
                 act_dtype=act_dtype, tau=tau, w_gate=w_gate, w_up=w_up, w_down_t=w_down_t,
                 s_gate=s_gate, s_up=s_up, s_down=s_down, b=b, p1=p1, p2=p2, b_p=b_p,
                 name="lattice")


def make_lattice_tokens(d: int, count: int, act_dtype: str = "f16", seed: int = 2) -> np.ndarray:
    rng = _rng(seed, (98, d, count))
    return _ternary(rng, (count, d), 0.5).astype(_NP_DTYPE[act_dtype])
