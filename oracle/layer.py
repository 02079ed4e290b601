"""The multi-tenant LoRA layer over a low-precision base GEMM, unfused, in fp64.

Test infrastructure only (see ``oracle/__init__.py``).

Notation follows "Punica: Serving multiple LoRA finetuned LLM as one" (README,
Overview): W has shape [H1, H2], adapter i has A_i [H1, r_i] and B_i [r_i, H2],
and a batch X whose parts x_i map to adapter i gives

    Y = X@W + (x_1@A_1@B_1, ..., x_n@A_n@B_n).

The EpiLoRA abstract adds the setting: W is stored in 8-bit (FP8) or 4-bit form,
the GEMM is low-precision, and each tenant's up-projection is added to the GEMM's
output (its epilogue).  With a per-adapter scale s_a this is, per token t with
adapter a = a(t):

    y[t] = dequant(x[t] . W) + s_a * (x[t] @ A_a) @ B_a.

Storage (H1 = K, H2 = N; W is kept [N, K] so that MX blocks run along K):

* FP8:   W_q uint8 [N, K] e4m3fn codes, s_w float32 [N] (one scale per output
         channel).  dequant(x.W)[t, n] = s_w[n] * sum_k X[t,k] * e4m3(W_q[n,k]).
* MXFP4: W_q uint8 [N, K/2], element k of row n in the low nibble of byte k//2
         when k is even and in the high nibble when k is odd; W_sc uint8
         [N, K/32] e8m0 codes for each run of 32 k.  W[k, n] =
         e2m1(nibble) * 2^(W_sc[n, k//32] - 127).

X is the MXFP8 form of the bf16 activations (``mxquant``); the adapters read the
bf16 x itself and A, B are bf16.  The steps below run in the order of the
formula: base product, then each adapter's down- and up-projection, then the sum.

The EpiLoRA abstract also names an engine variant that keeps the activations in
16 bits (to narrow the mismatch between generator and trainer).  There the base
product reads x itself: ``layer(..., act="bf16")`` gives dequant(x . W) with no
activation quantisation (``base_gemm_bf16``); everything else is unchanged.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from .codecs import bf16_to_f64, decode_e2m1, decode_e4m3fn
from .mxquant import MX_BLOCK, dequantize_mxfp8, quantize_mxfp8
from .segments import build_segments

# value of every e4m3fn code, from the decoder (NaN codes included)
_E4M3_VALUES = decode_e4m3fn(np.arange(256, dtype=np.uint8))
_E2M1_VALUES = decode_e2m1(np.arange(16))


@dataclass
class LowpWeight:
    """A base weight in one of the two formats.  ``fmt`` is "fp8" or "mxfp4"."""

    fmt: str
    q: np.ndarray          # uint8 [N, K] (fp8) or [N, K/2] (mxfp4)
    scale: np.ndarray      # float32 [N] (fp8) or uint8 [N, K/32] (mxfp4)

    @property
    def N(self) -> int:
        return int(self.q.shape[0])

    @property
    def K(self) -> int:
        return int(self.q.shape[1] * (1 if self.fmt == "fp8" else 2))


def dequant_weight(w: LowpWeight):
    """Return ``(Wd, col_scale)``: Wd float64 [N, K] exact, col_scale float64 [N] or None.

    For FP8 the per-channel scale is returned separately and is not folded into
    Wd, so that the K-sum below runs on exact dyadic values and the channel scale
    is applied once to the finished sum.
    """
    if w.fmt == "fp8":
        Wd = _E4M3_VALUES[np.asarray(w.q, dtype=np.uint8)]
        return Wd, np.asarray(w.scale, dtype=np.float32).astype(np.float64)
    if w.fmt == "mxfp4":
        q = np.asarray(w.q, dtype=np.uint8)
        N, half = q.shape
        nib = np.empty((N, half * 2), dtype=np.uint8)
        nib[:, 0::2] = q & 0xF
        nib[:, 1::2] = q >> 4
        vals = _E2M1_VALUES[nib].reshape(N, -1, MX_BLOCK)
        E = np.asarray(w.scale, dtype=np.int64) - 127
        return np.ldexp(vals, E[..., None].astype(np.int32)).reshape(N, -1), None
    raise ValueError(f"unknown weight format {w.fmt!r}")


def _weight_quantum_exp(w: LowpWeight) -> np.ndarray:
    """log2 of a power of two that divides every dequantised W element of row n."""
    if w.fmt == "fp8":
        return np.full(w.N, -9, dtype=np.int64)          # e4m3 grid step 2^-9
    E = np.asarray(w.scale, dtype=np.int64) - 127
    return -1 + E.min(axis=1)                              # e2m1 grid step 2^-1


def _exact_products_sum(X, Wd, qx, qw):
    """X @ Wd.T in float64, exact where a sufficient condition holds, else math.fsum.

    Every product X[t,k]*Wd[n,k] is a multiple of u = 2^(qx[t] + qw[n]) and has few
    significant bits; if sum_k |X[t,k] Wd[n,k]| < 2^52 u every partial sum is an
    exactly representable multiple of u, so the matmul is exact in any order.
    Entries that fail the test are recomputed with ``math.fsum`` (correctly rounded).
    """
    S = X @ Wd.T
    bound = np.abs(X) @ np.abs(Wd).T
    limit = np.ldexp(1.0, (52 + qx[:, None] + qw[None, :]).astype(np.int32))
    for t, n in np.argwhere(~(bound < limit)):
        S[t, n] = math.fsum(X[t] * Wd[n])
    return S


def base_gemm(x_q, x_sc, w: LowpWeight) -> np.ndarray:
    """dequant(X . W): float64 [T, N] from MXFP8 activations and a low-precision W.

    Every product X[t,k]*W[k,n] has at most 8 significant bits and is a multiple
    of u = 2^(qx[t] + qw[n]), where 2^qx and 2^qw divide every element of row t of
    X and row n of W.  If sum_k |X[t,k] W[k,n]| < 2^52 u, every partial sum is an
    exactly representable multiple of u, so the fp64 matmul is exact in any
    summation order.  This is checked at run time; entries that fail it are
    recomputed with ``math.fsum`` (correctly rounded).  The FP8 channel scale is
    then applied once.
    """
    X = dequantize_mxfp8(x_q, x_sc)
    Wd, col_scale = dequant_weight(w)
    if X.shape[1] != Wd.shape[1]:
        raise ValueError("K mismatch between activations and weight")
    qx = -9 + (np.asarray(x_sc, dtype=np.int64) - 127).min(axis=1) if X.shape[1] else np.zeros(X.shape[0], np.int64)
    S = _exact_products_sum(X, Wd, qx, _weight_quantum_exp(w))
    if col_scale is not None:
        S = S * col_scale[None, :]
    return S


def base_gemm_bf16(x_bits, w: LowpWeight) -> np.ndarray:
    """dequant(x . W) with the bf16 activations used as they are (16-bit variant).

    A bf16 value m * 2^e (0.5 <= |m| < 1) has at most 8 significant bits, so it is a
    multiple of 2^(e-8); a row of x is a multiple of 2^qx[t] with qx[t] the least
    such exponent over its nonzero entries.  The same exactness test as
    ``base_gemm`` applies; the FP8 channel scale is applied once to the sum.
    """
    x = bf16_to_f64(np.asarray(x_bits, dtype=np.uint16))
    Wd, col_scale = dequant_weight(w)
    if x.shape[1] != Wd.shape[1]:
        raise ValueError("K mismatch between activations and weight")
    _, e = np.frexp(x)
    e = np.where(x != 0, e.astype(np.int64) - 8, np.iinfo(np.int32).max)
    qx = e.min(axis=1) if x.shape[1] else np.zeros(x.shape[0], np.int64)
    qx = np.where(qx == np.iinfo(np.int32).max, 0, qx)     # all-zero row: any quantum
    S = _exact_products_sum(x, Wd, qx, _weight_quantum_exp(w))
    if col_scale is not None:
        S = S * col_scale[None, :]
    return S


def lora_terms(x_bits, A, B, scale, seg_indptr, sorted_tok, r_max: int):
    """Per-segment adapter terms: returns ``(t, y_lora)``.

    For each adapter a with a non-empty segment R_a (token indices in stable
    order): t[R_a, :r_a] = x[R_a] @ A_a and y_lora[R_a] = s_a * t[R_a, :r_a] @ B_a.
    ``t`` is float64 [T, r_max] in original token order, zero beyond r_a.
    """
    x = bf16_to_f64(x_bits)
    T = x.shape[0]
    n_ad = len(A)
    N = np.asarray(B[0]).shape[1] if n_ad else 0
    t = np.zeros((T, r_max), dtype=np.float64)
    y = np.zeros((T, N), dtype=np.float64)
    for a in range(n_ad):
        R = np.asarray(sorted_tok[seg_indptr[a]:seg_indptr[a + 1]], dtype=np.int64)
        if R.size == 0:
            continue
        Aa = bf16_to_f64(A[a])                 # [K, r_a]
        Ba = bf16_to_f64(B[a])                 # [r_a, N]
        r = Aa.shape[1]
        ta = x[R] @ Aa                         # down-projection
        t[R, :r] = ta
        y[R] = float(np.float32(scale[a])) * (ta @ Ba)   # up-projection, scaled
    return t, y


def layer(x_bits, w: LowpWeight, A, B, scale, adapter_id, act: str = "mxfp8"):
    """The whole layer, unfused.  Returns a dict of float64 / integer arrays.

    Keys: ``y`` (= y_base + y_lora), ``y_base``, ``y_lora``, ``t``, ``x_q``, ``x_sc``,
    ``seg_indptr``, ``sorted_tok``.  ``act`` is "mxfp8" (the base product reads the
    MXFP8 form of x) or "bf16" (it reads x itself; ``x_q`` and ``x_sc`` are then None).

    ``x_bits`` uint16 [T, K] bf16; ``A``/``B`` lists of bf16 (uint16) arrays
    [K, r_a] / [r_a, N]; ``scale`` float32 [n_adapters]; ``adapter_id`` int [T].
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    n_ad = len(A)
    seg_indptr, sorted_tok = build_segments(adapter_id, n_ad)
    if act == "mxfp8":
        x_q, x_sc = quantize_mxfp8(x_bits)
        y_base = base_gemm(x_q, x_sc, w)
    elif act == "bf16":
        x_q = x_sc = None
        y_base = base_gemm_bf16(x_bits, w)
    else:
        raise ValueError(f"unknown activation form {act!r}")
    r_max = max(int(np.asarray(a).shape[1]) for a in A)
    t, y_lora = lora_terms(x_bits, A, B, np.asarray(scale, dtype=np.float32), seg_indptr, sorted_tok, r_max)
    return {
        "y": y_base + y_lora,
        "y_base": y_base,
        "y_lora": y_lora,
        "t": t,
        "x_q": x_q,
        "x_sc": x_sc,
        "seg_indptr": seg_indptr,
        "sorted_tok": sorted_tok,
    }
