"""Plain float64 CPU oracle of the activation-sparse ReLU FFN decode step.

Test infrastructure: imported only by the tests, the smoke check and the
benchmark's CPU-baseline leg.  Shares no code with the GPU library.

What it computes, and where the PowerInfer pages define it:

* FFN(x) = sigma(x W1) (.) (x W2) W3 -- paper explainer (0h-n0.github.io,
  "PowerInfer - コンシューマGPUでの高速LLM推論エンジン"), section "ニューロン
  活性化のべき乗則分布" (power-law activation), FFN equation.  W1 is the gate,
  W2 the up projection, W3 the down projection, x a row vector.  sigma is
  ReLU: the project page ("使いやすさと互換性", "サポートするモデル") and the
  paper summary ("Limitations") make ReLU-sparse models the premise; the
  explainer's "SiLU" aside is read as a generic example.  A non-gated FFN is
  the same equation with the up projection alone under the ReLU.
* Predictor a_hat = sigmoid(x W_p + b_p), neuron i kept when a_hat_i > tau --
  explainer, section "活性化予測器" (activation predictor), predictor equation.
  The same section and the hybrid-architecture diagram call the predictor a
  small MLP; it is taken as a two-layer MLP of rank r with a ReLU hidden layer:
  z = max(x P1^T, 0) P2^T + b_p.  sigmoid(z) > tau is evaluated as
  z > log(tau / (1 - tau)) (the same set; no sigmoid is ever rounded).
* Only the predicted neurons are computed -- explainer, section "GPU-CPUハイブ
  リッドアーキテクチャ", inference flow steps 1-2; paper summary,
  "Methodology" (neuron-aware sparse operators work neuron by neuron).  The
  real ReLU is still applied to every computed neuron, so a predicted neuron
  whose pre-activation is negative contributes zero.
* int4 weights -- project page, "RTX 2080Ti性能（INT4量子化）"; paper summary,
  "Key Results" (quantized OPT-175B).  The pages give no format; the one used
  is signed 4-bit, two per byte (low nibble = even element), one fp16 scale per
  32 consecutive elements of a neuron row, value = q * s.

Batches of B tokens share one mask: the union of the per-token masks.
"""

from __future__ import annotations

import math
from typing import Optional

import numpy as np

UNIT_ROUNDOFF_F32 = 2.0 ** -24
GUARD_SAFETY = 2.0


# ----------------------------------------------------------------------------
# Weight decoding
# ----------------------------------------------------------------------------

def dequant_q4g32(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Decode packed int4 group-32 rows to float64.

    q: uint8 [rows][cols/2]; byte j holds element 2j in bits 0-3 and element
    2j+1 in bits 4-7, each a 4-bit two's complement integer in [-8, 7].
    s: fp16 [rows][cols/32]; element k of a row is q_k * s[k // 32].
    """
    q = np.asarray(q, dtype=np.uint8)
    rows, half = q.shape
    lo = (q & 0x0F).astype(np.int64)
    hi = (q >> 4).astype(np.int64)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    vals = np.empty((rows, 2 * half), dtype=np.float64)
    vals[:, 0::2] = lo
    vals[:, 1::2] = hi
    scales = np.asarray(s).astype(np.float64)
    if scales.shape != (rows, (2 * half) // 32):
        raise ValueError("scale shape does not match [rows][cols/32]")
    return vals * np.repeat(scales, 32, axis=1)


def dense_weights(w: np.ndarray, s: Optional[np.ndarray] = None) -> np.ndarray:
    """Stored weights (f32, f16, or packed int4 with scales) as float64."""
    if s is None:
        return np.asarray(w).astype(np.float64)
    return dequant_q4g32(w, s)


def _f64(a) -> np.ndarray:
    return np.atleast_2d(np.asarray(a).astype(np.float64))


# ----------------------------------------------------------------------------
# Predictor (explainer, "活性化予測器")
# ----------------------------------------------------------------------------

def predictor_hidden(x, p1) -> np.ndarray:
    """h = max(x P1^T, 0); x [B][d], P1 [r][d] -> [B][r]."""
    return np.maximum(_f64(x) @ _f64(p1).T, 0.0)


def predictor_logits(x, p1, p2, b_p) -> np.ndarray:
    """z = max(x P1^T, 0) P2^T + b_p; P2 [n][r], b_p [n] -> [B][n]."""
    return predictor_hidden(x, p1) @ _f64(p2).T + np.asarray(b_p).astype(np.float64)


def threshold_logit(tau: float) -> float:
    """sigmoid(z) > tau  <=>  z > log(tau / (1 - tau))."""
    if not (0.0 < tau < 1.0):
        raise ValueError("tau must lie in (0, 1)")
    return math.log(tau / (1.0 - tau))


def predicted_mask(z, tau: float) -> np.ndarray:
    """Per-token predicted mask, strict: z_i > logit(tau).  z == logit(tau) is inactive."""
    return np.asarray(z, dtype=np.float64) > threshold_logit(tau)


# ----------------------------------------------------------------------------
# FFN (explainer, "ニューロン活性化のべき乗則分布", FFN equation)
# ----------------------------------------------------------------------------

def pre_activations(x, w_gate, w_up, b, gated: bool):
    """Gated: g = x W_gate^T + b, u = x W_up^T.  Non-gated: g = x W_up^T + b, u = 1.

    Weights are neuron-major float64 [n][d]; returns (g, u), each [B][n].
    """
    xx = _f64(x)
    bb = np.asarray(b).astype(np.float64)
    if gated:
        g = xx @ np.asarray(w_gate, dtype=np.float64).T + bb
        u = xx @ np.asarray(w_up, dtype=np.float64).T
    else:
        g = xx @ np.asarray(w_up, dtype=np.float64).T + bb
        u = np.ones_like(g)
    return g, u


def activations(g, u) -> np.ndarray:
    """a = ReLU(g) (.) u."""
    return np.maximum(np.asarray(g, dtype=np.float64), 0.0) * np.asarray(u, dtype=np.float64)


def exact_mask(g) -> np.ndarray:
    """Neurons whose ReLU output is non-zero: g > 0 (per token)."""
    return np.asarray(g, dtype=np.float64) > 0.0


def union_mask(m) -> np.ndarray:
    """One mask for the whole batch: neuron i is computed if any token selects it."""
    return np.atleast_2d(np.asarray(m, dtype=bool)).any(axis=0)


def compact(mask):
    """Ascending int32 indices of the selected neurons, and their count."""
    idx = np.flatnonzero(np.asarray(mask, dtype=bool)).astype(np.int32)
    return idx, int(idx.size)


def down_projection(a, w_down_t, idx) -> np.ndarray:
    """y_t = sum over i in idx of a_t[i] * W_downT[i, :]  ([B][n], [n][d] -> [B][d])."""
    aa = _f64(a)
    idx = np.asarray(idx, dtype=np.int64)
    w = np.asarray(w_down_t, dtype=np.float64)
    if idx.size == 0:
        return np.zeros((aa.shape[0], w.shape[1]), dtype=np.float64)
    return aa[:, idx] @ w[idx, :]


def round_to_act(y, act_dtype: str) -> np.ndarray:
    """Round once, to nearest even, to the activation dtype."""
    return np.asarray(y, dtype=np.float64).astype({"f32": np.float32, "f16": np.float16}[act_dtype])


def _layer_weights(layer):
    w_gate = dense_weights(layer.w_gate, layer.s_gate) if layer.gated else None
    w_up = dense_weights(layer.w_up, layer.s_up)
    w_down_t = dense_weights(layer.w_down_t, layer.s_down)
    return w_gate, w_up, w_down_t


def hot_mask(n: int, hot=None) -> np.ndarray:
    """The always-computed hot neurons as a boolean mask over the n neurons (hot: a boolean mask
    or a list of neuron ids; None is the empty set).

    The paper explainer's offline profiling (section "オフラインプロファイリング") counts how often
    each neuron fires on calibration inputs and sorts the neurons by that count; the project page
    ("コア技術原理") and the paper summary ("Key Results") describe the few hot neurons that fire
    on almost every input.  The hot set is computed on every token without consulting the
    predictor.
    """
    m = np.zeros(n, dtype=bool)
    if hot is None:
        return m
    hot = np.asarray(hot)
    if hot.dtype == bool:
        if hot.shape != (n,):
            raise ValueError("a hot mask must have one entry per neuron")
        return hot.copy()
    m[hot.astype(np.int64)] = True
    return m


def forward(layer, x, mode: str = "predicted", weights=None, hot=None) -> dict:
    """The whole step for a batch x [B][d]: mask -> indices -> activations -> output.

    mode: "predicted" (predictor mask), "exact" (mask = ReLU support), "dense" (all
    neurons).  `weights` may pass pre-decoded (w_gate, w_up, w_down_t) float64.
    hot (predicted mode): neurons selected whatever the predictor says (the profile's hot set,
    as a boolean mask or id list); the predictor decides the rest.
    Returns idx, count, y64 (float64 [B][d]) and y (rounded to the act dtype),
    plus the intermediate g, u, a and (predicted mode) z.
    """
    xx = _f64(x)
    w_gate, w_up, w_down_t = weights if weights is not None else _layer_weights(layer)
    g, u = pre_activations(xx, w_gate, w_up, layer.b, layer.gated)
    a = activations(g, u)
    out = {"g": g, "u": u, "a": a}
    if mode == "predicted":
        z = predictor_logits(xx, layer.p1, layer.p2, layer.b_p)
        out["z"] = z
        mask = union_mask(predicted_mask(z, layer.tau)) | hot_mask(layer.d_ffn, hot)
    elif mode == "exact":
        mask = union_mask(exact_mask(g))
    elif mode == "dense":
        mask = np.ones(layer.d_ffn, dtype=bool)
    else:
        raise ValueError(f"unknown mode {mode!r}")
    idx, count = compact(mask)
    y64 = down_projection(a, w_down_t, idx)
    out.update(mask=mask, idx=idx, count=count, y64=y64, y=round_to_act(y64, layer.act_dtype))
    return out


def forward_masked(layer, x, idx, weights=None) -> dict:
    """The sparse operator on a caller-given ascending index list.

    Only the listed neurons' rows are decoded and used: y_t = sum over i in idx
    of ReLU(g_t[i]) u_t[i] W_downT[i].  Returns a (for the listed neurons, in
    list order), y64 and y.
    """
    xx = _f64(x)
    idx = np.asarray(idx, dtype=np.int64)

    def rows(w, s):
        if w is None:
            return None
        return dense_weights(np.asarray(w)[idx], None if s is None else np.asarray(s)[idx])

    if weights is not None:
        w_gate, w_up, w_down_t = (None if w is None else np.asarray(w)[idx] for w in weights)
    else:
        w_gate = rows(layer.w_gate, layer.s_gate) if layer.gated else None
        w_up = rows(layer.w_up, layer.s_up)
        w_down_t = rows(layer.w_down_t, layer.s_down)
    g, u = pre_activations(xx, w_gate, w_up, np.asarray(layer.b)[idx], layer.gated)
    a = activations(g, u)
    y64 = down_projection(a, w_down_t, np.arange(idx.size))
    if idx.size == 0:
        y64 = np.zeros((xx.shape[0], xx.shape[1]), dtype=np.float64)
    return {"g": g, "u": u, "a": a, "y64": y64, "y": round_to_act(y64, layer.act_dtype)}


# ----------------------------------------------------------------------------
# Guard bands: how far an fp32 evaluation of a logit can be from the exact one.
# A decision is compared only outside the band; inside it either side is right.
# ----------------------------------------------------------------------------

def gamma(m: int, u: float = UNIT_ROUNDOFF_F32) -> float:
    """gamma_m = m u / (1 - m u): bound on the relative error of m rounded operations."""
    return m * u / (1.0 - m * u)


def guard_band_exact(x, w_rows, b) -> np.ndarray:
    """Band for g_i = x . w_i + b_i evaluated in fp32 in any order: 2 gamma_{d+2}(|x|.|w_i| + |b_i|)."""
    xx = np.abs(_f64(x))
    w = np.abs(np.asarray(w_rows, dtype=np.float64))
    d = w.shape[1]
    return GUARD_SAFETY * gamma(d + 2) * (xx @ w.T + np.abs(np.asarray(b, dtype=np.float64)))


def guard_band_predictor(x, p1, p2, b_p) -> np.ndarray:
    """Band for z_i with h and z both accumulated in fp32.

    |dz_i| <= gamma_{r+2}(|P2_i|.|h| + |b_p,i|) + |P2_i|.|dh|, |dh_j| <= gamma_{d+2} |x|.|P1_j|.
    """
    xx = _f64(x)
    p1a = np.asarray(p1, dtype=np.float64)
    p2a = np.abs(np.asarray(p2, dtype=np.float64))
    d, r = p1a.shape[1], p1a.shape[0]
    h = np.maximum(xx @ p1a.T, 0.0)
    dh = gamma(d + 2) * (np.abs(xx) @ np.abs(p1a).T)
    bound = gamma(r + 2) * (h @ p2a.T + np.abs(np.asarray(b_p, dtype=np.float64))) + dh @ p2a.T
    return GUARD_SAFETY * bound


# ----------------------------------------------------------------------------
# Probabilistic guard bands (Higham and Mary, "A New Approach to Probabilistic
# Rounding Error Analysis", SIAM J. Sci. Comput. 41(5), 2019): rounding errors
# are modelled as independent, mean-zero random variables, each at most u times
# the value being rounded.  To first order, the error of an fp32 value built
# from m roundings is then a sum of m independent bounded mean-zero terms, and
# Hoeffding's inequality bounds it by lambda * u * sqrt(sum of squared term
# bounds) except with probability 2 exp(-lambda^2 / 2).  Every partial sum of a
# dot product, in any order, is at most the sum of the absolute terms, which
# bounds each term.  For the predictor logit all roundings (those of h, carried
# through P2, and those of z's own dot product) are bounded together.
# ----------------------------------------------------------------------------

PROB_LAMBDA = 10.0   # 2 exp(-50) ~ 4e-22 per value: no realistic test meets a miss


def _rounding_events(k: int) -> int:
    """Roundings an fp32 dot product of k terms plus a bias may take: one per product and one per
    addition (products of two fp16 values are exact in fp32; counting them is harmless)."""
    return 2 * k + 2


def prob_band_exact(x, w_rows, b, lam: float = PROB_LAMBDA) -> np.ndarray:
    """Band for g_i = x . w_i + b_i in fp32: lambda u sqrt(m) (|x|.|w_i| + |b_i|), plus the
    second-order term (m u)^2 times the same magnitude."""
    xx = np.abs(_f64(x))
    w = np.abs(np.asarray(w_rows, dtype=np.float64))
    m = _rounding_events(w.shape[1])
    mag = xx @ w.T + np.abs(np.asarray(b, dtype=np.float64))
    u = UNIT_ROUNDOFF_F32
    return (lam * u * math.sqrt(m) + (m * u) ** 2) * mag


def prob_band_predictor(x, p1, p2, b_p, lam: float = PROB_LAMBDA) -> np.ndarray:
    """Band for z_i = ReLU(x P1^T) P2_i + b_p,i with h and z accumulated in fp32.

    First order: z_hat - z = sum_j P2_ij dh_j + e_i, dh_j a sum of m_h roundings each at most
    u A_j (A_j = |x|.|P1_j|), e_i a sum of m_z roundings each at most u C_i
    (C_i = |P2_i|.|h| + |b_p,i|).  Hoeffding over all of them:
    lambda u sqrt(m_h sum_j P2_ij^2 A_j^2 + m_z C_i^2).  Second order: (m_h u)^2 |P2_i|.A
    + (m_z u)^2 C_i.
    """
    xx = _f64(x)
    p1a = np.asarray(p1, dtype=np.float64)
    p2a = np.asarray(p2, dtype=np.float64)
    d, r = p1a.shape[1], p1a.shape[0]
    m_h, m_z = _rounding_events(d), _rounding_events(r)
    u = UNIT_ROUNDOFF_F32
    A = np.abs(xx) @ np.abs(p1a).T                          # [B][r]
    h = np.maximum(xx @ p1a.T, 0.0)
    C = h @ np.abs(p2a).T + np.abs(np.asarray(b_p, dtype=np.float64))
    first = lam * u * np.sqrt(m_h * ((A * A) @ (p2a * p2a).T) + m_z * C * C)
    second = (m_h * u) ** 2 * (A @ np.abs(p2a).T) + (m_z * u) ** 2 * C
    return first + second


def certain_union(values, band, threshold: float = 0.0):
    """(certainly_on, certainly_off) for the batch-union decision values > threshold."""
    v = _f64(values)
    g = _f64(band)
    on = (v - g > threshold).any(axis=0)
    off = (v + g < threshold).all(axis=0)
    return on, off
