"""Brute-force reference for tiny inputs (numpy, float64), written independently
of the oracle: it runs EVERY expert on EVERY token and weights each result by
the dense gate vector, i.e. y = sum over all experts i of g_i * E_i(x), the
weighted sum of page 1 ("Mixture of Experts (MoE) 12段階極小ビジュアル解剖シミュレーター",
STEP 12), with g the softmax of the -inf-masked score vector (STEP 5-6).

It has no notion of capacity, slots or dispatch, so it equals the layer only
when nothing is dropped. Ranking is decided on float32-rounded scores (the
pages' router runs in full precision, nanoMoE slide 11), ties to the lower
expert index, using numpy's stable argsort.

The nanoMoE slides' expert variant (slide 32: bias after each projection,
GELU between them) is covered the same way: biases are added to every
expert's product and GELU is x * Phi(x), with Phi built from Python's scalar
math.erf.
"""
import math

import numpy as np


def dense_gates(x64, wg64, noise64, k):
    s = x64 @ wg64.T
    if noise64 is not None:
        s = s + noise64
    s32 = s.astype(np.float32).astype(np.float64)
    N, E = s32.shape
    order = np.argsort(-s32, axis=1, kind="stable")[:, :k]
    masked = np.full((N, E), -np.inf)
    rows = np.arange(N)[:, None]
    masked[rows, order] = s32[rows, order]
    m = masked.max(axis=1, keepdims=True)
    ex = np.exp(masked - m)
    return ex / ex.sum(axis=1, keepdims=True), order


_erf = np.vectorize(math.erf)


def expert_all_tokens(x64, wup64, wdown64, act="relu", bup=None, bdown=None):
    z = x64 @ wup64.T
    if bup is not None:
        z = z + bup
    h = np.maximum(z, 0.0) if act == "relu" else z * 0.5 * (1.0 + _erf(z / math.sqrt(2.0)))
    y = h @ wdown64.T
    if bdown is not None:
        y = y + bdown
    return y


def layer(x64, wg64, noise64, k, wups, wdowns, act="relu", bups=None, bdowns=None):
    G, order = dense_gates(x64, wg64, noise64, k)
    out = np.zeros_like(x64)
    for e in range(wg64.shape[0]):
        out += G[:, e:e + 1] * expert_all_tokens(
            x64, wups[e], wdowns[e], act,
            None if bups is None else bups[e], None if bdowns is None else bdowns[e])
    return out, G, order
