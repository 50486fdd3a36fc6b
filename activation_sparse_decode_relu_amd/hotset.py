"""Offline profiling and the hot set (host-side deployment tooling).

The paper explainer's offline profiling (section "オフラインプロファイリング") runs the model on
calibration inputs, counts how often each neuron fires, and sorts the neurons by that count;
the project page ("コア技術原理") and the paper summary ("Key Results") describe the few hot
neurons that fire on almost every input.  On one GPU there is nothing to place on a second
device, so the profile marks the neurons that fired on (almost) every calibration token as the
layer's hot set, which the library computes on every token without consulting the predictor
(pi_ffn_set_hot).  The neurons stay where they are: gathering the hot ones at the front of the
layer would hand all of them to a few waves and put their rows on a fixed stride.

The counting runs the library's exact-ReLU mode on the calibration tokens (the activations the
layer really produces); the rest is host bookkeeping on numpy arrays.
"""

from __future__ import annotations

import numpy as np


def firing_counts(handle, tokens) -> np.ndarray:
    """How many of the calibration tokens (device tensor [T][d]) fire each neuron, from the
    library's exact-ReLU mode, one token at a time."""
    import torch
    n = handle.desc.d_ffn
    y = torch.empty((1, tokens.shape[1]), dtype=tokens.dtype, device=tokens.device)
    idx = torch.empty(n, dtype=torch.int32, device=tokens.device)
    count = torch.empty(1, dtype=torch.int32, device=tokens.device)
    counts = np.zeros(n, dtype=np.int64)
    for t in range(tokens.shape[0]):
        handle.forward(tokens[t:t + 1], y, "exact", idx, count)
        c = int(count.item())
        counts += np.bincount(idx[:c].cpu().numpy(), minlength=n)
    return counts


def hot_set(counts, n_tokens: int, hot_fraction: float = 0.99) -> np.ndarray:
    """Boolean mask of the neurons that fired on at least hot_fraction of the n_tokens tokens."""
    return np.asarray(counts) >= hot_fraction * n_tokens


def hot_words(mask) -> np.ndarray:
    """The library's bit set: uint32 words, bit b of word w = neuron 32 w + b."""
    mask = np.asarray(mask, dtype=bool)
    padded = np.zeros((mask.size + 31) // 32 * 32, dtype=bool)
    padded[:mask.size] = mask
    bits = padded.reshape(-1, 32).astype(np.uint64) << np.arange(32, dtype=np.uint64)
    return bits.sum(axis=1).astype(np.uint32)
