"""CPU oracle for the dilated depthwise 1-D convolution and the fused
depthwise + pointwise module -- test infrastructure.

Only ``tests/`` and ``bench.py``'s CPU-baseline leg may import this module; the
product path never does.

The operation is the one the JAX issue page on grouped and dilated
convolutions benchmarks (its reproduction script: ``depthwise`` with
``feature_group_count`` equal to the channel count, "NTC" input, "TIO" kernel
with one input feature per group, stride 1, VALID padding, ``rhs_dilation``
d): for every batch b, output step t < T and channel c,

    y[b, t, c] = sum_{k < K} w[k, c] * x[b, t + k*d, c],

with x of length T + d*(K - 1).  Written out here in fp64 as a sum of K
shifted, scaled copies of the input, in the order k = 0, 1, ..., K-1.
"""
from __future__ import annotations

import numpy as np


def dwconv1d(x: np.ndarray, w: np.ndarray, dilation: int) -> np.ndarray:
    """x [B][T + d(K-1)][C], w [K][C] -> y [B][T][C] (float64)."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    K, C = w.shape
    B, L, C2 = x.shape
    assert C2 == C and dilation >= 1
    T = L - dilation * (K - 1)
    assert T >= 0
    y = np.zeros((B, T, C), np.float64)
    for k in range(K):
        y += w[k][None, None, :] * x[:, k * dilation:k * dilation + T, :]
    return y


def dwpw1d(x: np.ndarray, w_dw: np.ndarray, w_pw: np.ndarray, dilation: int) -> np.ndarray:
    """Depthwise then pointwise, the pair the FCM abstract fuses: the dilated
    depthwise convolution above, then a 1x1 convolution mixing channels,
    z[b, t, o] = sum_c y[b, t, c] * w_pw[c, o] ("TIO" kernel with one tap).
    x [B][T + d(K-1)][C], w_dw [K][C], w_pw [C][O] -> z [B][T][O] (float64);
    the channel mix is one matrix product per batch."""
    y = dwconv1d(x, w_dw, dilation)
    return y @ np.asarray(w_pw, np.float64)
