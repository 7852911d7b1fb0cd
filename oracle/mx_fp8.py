"""MX-FP8 (E4M3 elements, one E8M0 power-of-two scale per 32 consecutive
values) quantization and the FP8 output projection, CPU, float64.

TEST INFRASTRUCTURE ONLY.  Only ``tests/`` may import this module; the HIP
library never imports it and shares no code with it.

The pages run the linear layers after the attention in FP8 (deepmagic blog
"生成比播放還快", section 實測數據: the 125.3 ms block uses FP8 linear layers)
without fixing the format.  The reading taken here is the OCP Microscaling
format MXFP8 (E4M3), which gfx950's scaled MFMA consumes directly: per block
of 32 values along the contraction,

  X   = floor(log2(max |v|)) - 8            (8 = exponent of E4M3's largest
                                             normal, 448 = 1.75 * 2^8)
  P_i = E4M3(v_i / 2^X)                     round to nearest, ties to even,
                                             magnitudes past 448 clamped to 448
  v_i ~ P_i * 2^X

with X stored biased by 127 (E8M0, so X >= -127); an all-zero block gets
X = 0.  E4M3 here
is the OCP format: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits,
subnormals down to 2^-9, largest finite 448, no infinities.
"""
from __future__ import annotations

import numpy as np

__all__ = ["E4M3_MAX", "round_e4m3", "mx_quantize", "mx_dequantize", "output_projection_mxfp8"]

E4M3_MAX = 448.0
BLOCK = 32


def round_e4m3(x) -> np.ndarray:
    """Round to the nearest E4M3 value (ties to even), clamping magnitudes
    past 448; float64 in, float64 out."""
    x = np.asarray(x, np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    # exponent of the binade, never below the normal minimum 2^-6 (subnormals
    # share the spacing 2^-9 of the lowest binade)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)
    step = 2.0 ** (e - 3)                    # 3 mantissa bits
    q = np.round(a / step) * step            # numpy rounds halves to even
    q = np.minimum(q, E4M3_MAX)
    return np.sign(x) * q


def mx_quantize(x, block: int = BLOCK):
    """Quantize along the last axis in blocks of ``block`` values.  Returns
    (elements as float64 E4M3 values, per-block exponents X as int)."""
    x = np.asarray(x, np.float64)
    assert x.shape[-1] % block == 0
    xb = x.reshape(x.shape[:-1] + (x.shape[-1] // block, block))
    amax = np.abs(xb).max(axis=-1)
    with np.errstate(divide="ignore"):
        X = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8, 0).astype(np.int64)
    X = np.maximum(X, -127)                 # E8M0 holds 2^-127 .. 2^127
    P = round_e4m3(xb / (2.0 ** X)[..., None])
    return P.reshape(x.shape), X


def mx_dequantize(P, X, block: int = BLOCK) -> np.ndarray:
    P = np.asarray(P, np.float64)
    Pb = P.reshape(P.shape[:-1] + (P.shape[-1] // block, block))
    return (Pb * (2.0 ** np.asarray(X, np.float64))[..., None]).reshape(P.shape)


def output_projection_mxfp8(x, w) -> np.ndarray:
    """y = Q(x) Q(w)^T with both operands MX-FP8 quantized along the
    contraction (x [..., K], w [N, K]): the exact product of the quantized
    values, as the FP8 projection computes it up to fp32 accumulation."""
    xq = mx_dequantize(*mx_quantize(x))
    wq = mx_dequantize(*mx_quantize(w))
    return xq @ wq.T
