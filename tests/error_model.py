"""Error model of the bfloat16 decode path, for tolerances that can fail.

The stated tolerance for bfloat16 keys and values with float32 accumulation
is an absolute 2e-2.  At the benchmark lengths an output row is small
(|out| shrinks like sqrt(e / L) for N(0, 1) data), so 2e-2 alone would pass
an all-zero row at L = 131,072 or a dropped 32-token step at L = 4,096.
The parity tests therefore also check each element against a bound derived
from what the kernels round:

* bfloat16 products of bfloat16 inputs are exact in float32, and the
  float32 sums of 128 of them (scores) and of the softmax terms move an
  output by ~1e-6 at most: covered by the floor ``A_FLOOR``;
* the probabilities p_i (float32, at most 1 after the running maximum) are
  rounded to nearest-even bfloat16 for the PV product, a relative error
  eps_i with |eps_i| <= U = 2^-8, while the softmax sum uses the unrounded
  p_i.  The output moves by sum_i eps_i w_i v_i (w_i = p_i / sum p, the
  normalised weights), whose spread is (U / sqrt(3)) * r with
  r = sqrt(sum_i w_i^2 v_i^2); ``Z`` = 8 of those spreads bound it (and
  Z / sqrt(3) > 1 also covers the worst case of one dominant term);
* the output is rounded to nearest-even bfloat16: at most U * |out|.

bound[h, d] = U * |ref[h, d]| + (1 + U) * Z * (U / sqrt(3)) * r[h, d] + A_FLOOR

``tests/test_error_model.py`` shows on the CPU, at the workloads' own
lengths, that a correctly rounded result stays inside this bound while one
dropped or double-counted 32-token step, or one dropped 512-token
partition, leaves it.
"""
from __future__ import annotations

import math

import numpy as np

U = 2.0 ** -8  # unit roundoff of bfloat16 (8 significant bits)
Z = 8.0
A_FLOOR = 1e-5


def weights_and_spread(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """For one sequence (q [Hq, D], K/V [L, Hkv, D], float64): the exact
    output [Hq, D] and r[h, d] = sqrt(sum_i w_i^2 v_i[d]^2) [Hq, D]."""
    Hq, D = q.shape
    L, Hkv, _ = K.shape
    G = Hq // Hkv
    out = np.zeros((Hq, D))
    r = np.zeros((Hq, D))
    if L == 0:
        return out, r
    for g in range(Hkv):
        Kg = np.ascontiguousarray(K[:, g, :])
        Vg = np.ascontiguousarray(V[:, g, :])
        S = scale * (q[g * G:(g + 1) * G] @ Kg.T)  # [G, L]
        E = np.exp(S - S.max(axis=1, keepdims=True))
        W = E / E.sum(axis=1, keepdims=True)
        out[g * G:(g + 1) * G] = W @ Vg
        r[g * G:(g + 1) * G] = np.sqrt((W * W) @ (Vg * Vg))
    return out, r


def bf16_bound(ref: np.ndarray, r: np.ndarray) -> np.ndarray:
    """Per-element bound on |kernel - exact| for bfloat16 keys/values."""
    return U * np.abs(ref) + (1.0 + U) * Z * (U / math.sqrt(3.0)) * r + A_FLOOR


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest-even bfloat16 -> float64 (via torch's conversion)."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)).to(torch.bfloat16).double().numpy()
