"""Plain fp64 reference for the steps on either side of the attention: the QKV
projection with rotary position encoding before it and the output projection after
it, with 8-bit weights.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Where this comes from
---------------------
The hotpaper.ai page "DuoAttention: Efficient Long-Context LLM Inference with
Retrieval and Streaming Heads" (abstract; the Korean sections on the technical approach
and the main results) states that the method combines with 8-bit weight quantization
and a 4-bit KV cache, and that Llama-3-8B then decodes 3.3M tokens on one A100.  The
pages give no weight format and say nothing of position encoding, so this module takes
the plainest readings:

* 8-bit weights: a linear layer's weight W [N, K] (output channel n, input feature k)
  is held as int8 codes c[n, k] in [-127, 127] and one fp32 scale s[n] per output
  channel; the layer computes y[m, n] = sum_k x[m, k] * c[n, k] * s[n] (weight-only
  quantization: activations stay in the I/O dtype).
* position encoding: the rotary encoding of the models the pages run (Llama-2 and
  Llama-3; RoFormer, Su et al. 2021, eq. 34 in the "rotate half" pairing those models
  use): within each head of size D, dims d and d + D/2 (d < D/2) form a pair that is
  rotated by the angle pos * theta_d, theta_d = base ** (-2 d / D), where pos is the
  token's absolute position; queries and keys are rotated, values are not.
* the fused QKV projection's output channels are the query heads, then the key heads,
  then the value heads, each head D consecutive channels.

Everything is float64: codes and scales are exact in float64, products are formed with
NumPy matrix products in float64, and the rotation uses float64 cos / sin.
"""

from __future__ import annotations

import numpy as np


def w8_linear(x: np.ndarray, codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """y[m, n] = sum_k x[m, k] * codes[n, k] * scales[n], in float64.

    x: [M, K] (any float dtype, upcast exactly); codes: [N, K] int8; scales: [N]."""
    xf = np.asarray(x, dtype=np.float64)
    w = np.asarray(codes, dtype=np.float64) * np.asarray(scales, dtype=np.float64)[:, None]
    return xf @ w.T


def rope_frequencies(D: int, base: float) -> np.ndarray:
    """theta_d = base ** (-2 d / D) for d in [0, D/2) (RoFormer's frequencies)."""
    d = np.arange(D // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * d / D)


def rope(x: np.ndarray, positions, base: float) -> np.ndarray:
    """Rotary encoding of x [n, H, D] (token n at absolute position positions[n]): for
    each head and d < D/2,
        out[d]       = x[d] cos(a) - x[d + D/2] sin(a)
        out[d + D/2] = x[d + D/2] cos(a) + x[d] sin(a),     a = pos * theta_d."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    h = D // 2
    a = np.asarray(positions, dtype=np.float64)[:, None] * rope_frequencies(D, base)[None, :]
    c = np.cos(a)[:, None, :]
    s = np.sin(a)[:, None, :]
    lo, hi = x[..., :h], x[..., h:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def qkv_rope(x: np.ndarray, codes: np.ndarray, scales: np.ndarray, Hq: int, Hkv: int, D: int, positions,
             base: float):
    """Fused QKV projection of tokens x [n, hidden] at the given absolute positions,
    then the rotary encoding of the query and key heads.  Returns (q [n, Hq, D],
    k [n, Hkv, D], v [n, Hkv, D]) in float64."""
    y = w8_linear(x, codes, scales)
    n = y.shape[0]
    q = y[:, :Hq * D].reshape(n, Hq, D)
    k = y[:, Hq * D:(Hq + Hkv) * D].reshape(n, Hkv, D)
    v = y[:, (Hq + Hkv) * D:].reshape(n, Hkv, D)
    return rope(q, positions, base), rope(k, positions, base), v
