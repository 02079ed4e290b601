"""MXFP8 quantisation of the layer's bf16 activations (oracle side).

Test infrastructure only (see ``oracle/__init__.py``).

The EpiLoRA abstract says the base GEMM runs in a low-precision format and that
an engine variant "keeps activations in 16 bits" -- so in the default engine the
activations entering the base GEMM are low-precision too.  The pages do not fix
the activation format; the reading taken here is MXFP8 (OCP Microscaling Formats
v1.0): each run of 32 consecutive elements along K of one token row shares one
e8m0 scale 2^E, and each element is stored as an e4m3fn code.  The rule, as the
MX spec gives it for e4m3 (largest element exponent 8):

    m = max |x| over the block
    E = floor(log2 m) - 8, clamped to [-127, 127]; E = -127 when m == 0
    scale code = E + 127
    element code = RNE_e4m3( clamp(x * 2^-E, -448, 448) )   (sign kept)

The scaling by 2^-E is exact, so the result is a pure function of the 32 inputs.
The LoRA down-projection does not use these codes: it reads the bf16 x.
"""

from __future__ import annotations

import numpy as np

from .codecs import E4M3_MAX, bf16_to_f64, decode_e4m3fn, encode_e4m3fn_rne

MX_BLOCK = 32
E4M3_EMAX = 8


def quantize_mxfp8(x_bits):
    """Quantise bf16 activations [T, K] (uint16 bits) to MXFP8.

    Returns ``(x_q, x_sc)``: e4m3fn codes uint8 [T, K] and e8m0 scale codes
    uint8 [T, K/32].  K must be a multiple of 32.
    """
    x = bf16_to_f64(x_bits)
    if x.ndim != 2 or x.shape[1] % MX_BLOCK:
        raise ValueError("x must be [T, K] with K a multiple of 32")
    T, K = x.shape
    xb = x.reshape(T, K // MX_BLOCK, MX_BLOCK)
    m = np.abs(xb).max(axis=2)
    _, e = np.frexp(np.where(m > 0, m, 1.0))          # m = f * 2^e, 0.5 <= f < 1
    floor_log2 = e.astype(np.int64) - 1
    E = np.where(m > 0, floor_log2 - E4M3_EMAX, -127)
    E = np.clip(E, -127, 127)
    v = np.ldexp(xb, (-E)[..., None].astype(np.int32))  # exact power-of-two scaling
    v = np.clip(v, -E4M3_MAX, E4M3_MAX)
    x_q = encode_e4m3fn_rne(v).reshape(T, K)
    x_sc = (E + 127).astype(np.uint8)
    return x_q, x_sc


def dequantize_mxfp8(x_q, x_sc) -> np.ndarray:
    """Exact float64 values of MXFP8 data: decode(code) * 2^(scale - 127)."""
    x_q = np.asarray(x_q, dtype=np.uint8)
    T, K = x_q.shape
    vals = decode_e4m3fn(x_q).reshape(T, K // MX_BLOCK, MX_BLOCK)
    E = np.asarray(x_sc, dtype=np.int64) - 127
    return np.ldexp(vals, E[..., None].astype(np.int32)).reshape(T, K)
