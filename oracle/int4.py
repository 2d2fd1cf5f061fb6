"""Reference int4 KV codec: per-token, per-head, group-128, asymmetric, fp16 scale/zero.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages state only that DuoAttention combines with a 4-bit KV cache (hotpaper.ai
page "DuoAttention: Efficient Long-Context LLM Inference with Retrieval and Streaming
Heads": abstract, which pairs the method with quantization for 3.3M-token decoding of
Llama-3-8B on one A100; and its key-contributions and main-results sections, which
name 8-bit weights with a 4-bit KV cache).  The format itself (one group per 128-value
vector, asymmetric, scale and zero stored as fp16) is the workload's stated format.
Where neither fixes a step, this module takes the plainest reading:

For each stored vector x (one token, one KV head, K or V; 128 bfloat16 values):

* mn = min x, mx = max x, in float32 (the bf16 -> fp32 upcast is exact);
* s = fp16_RN( fp32_RN( fp32_RN(mx - mn) / 15 ) ),  z = fp16_RN(mn);
* if s == 0 every code is 0; otherwise
  q_k = clamp( rint_half_even( fp32_RN( fp32_RN(x_k - z) / s ) ), 0, 15 );
* byte k of the packed row holds q_{2k} in its low nibble and q_{2k+1} in its high one;
* dequantised value: x_hat_k = fp32_RN(q_k * s + z).

q_k has 4 significant bits and s 11, so q_k * s is exact in float32: a fused
multiply-add and a multiply followed by an add give the same x_hat, which makes the
dequantised value a well-defined bit pattern.
"""

from __future__ import annotations

import numpy as np

GROUP = 128


def _bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _scale_fp16(s32: np.ndarray) -> np.ndarray:
    """The stored scale: the fp32 quotient rounded to nearest fp16."""
    return np.asarray(s32, dtype=np.float32).astype(np.float16)


def _zero_fp16(mn: np.ndarray) -> np.ndarray:
    """The stored zero: the vector's minimum rounded to nearest fp16."""
    return np.asarray(mn, dtype=np.float32).astype(np.float16)


def quantize(x_bf16_bits: np.ndarray):
    """Quantise bf16 vectors (uint16 bit patterns, last axis 128).

    Returns (codes uint8[..., 64], scale float16[...], zero float16[...])."""
    x = _bf16_to_f32(x_bf16_bits)
    if x.shape[-1] != GROUP:
        raise ValueError("int4 groups are 128 values")
    mn = x.min(axis=-1)
    mx = x.max(axis=-1)
    rng = (mx - mn).astype(np.float32)                       # fp32 subtract
    s32 = (rng / np.float32(15.0)).astype(np.float32)        # fp32 divide
    s16 = _scale_fp16(s32)                                   # RN to fp16
    z16 = _zero_fp16(mn)                                     # RN to fp16
    s = s16.astype(np.float32)[..., None]
    z = z16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = ((x - z).astype(np.float32) / s).astype(np.float32)
    q = np.clip(np.rint(t), 0, 15)
    q = np.where(s == 0, 0, q).astype(np.uint8)
    codes = (q[..., 0::2] | (q[..., 1::2] << np.uint8(4))).astype(np.uint8)
    return codes, s16, z16


def unpack(codes: np.ndarray) -> np.ndarray:
    """uint8[..., 64] packed codes -> uint8[..., 128] codes in element order."""
    codes = np.asarray(codes, dtype=np.uint8)
    q = np.empty(codes.shape[:-1] + (2 * codes.shape[-1],), dtype=np.uint8)
    q[..., 0::2] = codes & np.uint8(0x0F)
    q[..., 1::2] = codes >> np.uint8(4)
    return q


def dequantize(codes: np.ndarray, scale: np.ndarray, zero: np.ndarray) -> np.ndarray:
    """x_hat = fp32_RN(q * s + z), float32[..., 128]."""
    q = unpack(codes).astype(np.float32)
    s = np.asarray(scale, dtype=np.float16).astype(np.float32)[..., None]
    z = np.asarray(zero, dtype=np.float16).astype(np.float32)[..., None]
    prod = (q * s).astype(np.float32)   # exact: 4-bit times 11-bit significand
    return (prod + z).astype(np.float32)
