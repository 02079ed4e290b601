"""Gradients of the multi-tenant LoRA layer on a frozen low-precision base, unfused, in fp64.

Test infrastructure only (see ``oracle/__init__.py``).

The EpiLoRA abstract: the same low-precision base also trains -- a LoRA trainer computes on
the engine's FP8 weights (no 16-bit copy of W), and keeps activations in 16 bits.  The layer
being trained is therefore the 16-bit-activation form of ``layer.layer(..., act="bf16")``:
per token t with adapter a = a(t),

    y[t] = x[t] . W_d + s_a (x[t] A_a) B_a,

with W_d the dequantised base weight (frozen) and A_a [K, r_a], B_a [r_a, N] trained.  Given
the gradient dY of a loss with respect to y (bf16, as a 16-bit engine passes it), the chain
rule gives, over the tokens R_a of adapter a (the segment of "Punica" README, Overview):

    u[t]  = dY[t] B_a^T                       [r_a]   (the up-projection transposed)
    dX[t] = dY[t] W_d^T + s_a u[t] A_a^T      [K]
    dA_a  = s_a sum_{t in R_a} x[t]^T u[t]    [K, r_a]
    dB_a  = s_a sum_{t in R_a} t_a[t]^T dY[t] [r_a, N],  t_a[t] = x[t] A_a

The steps below follow that order; everything is fp64 from the bf16 inputs and the exactly
dequantised W.  Tokens whose adapter id is outside [0, n) are an error, as in the forward.
"""

from __future__ import annotations

import numpy as np

from .codecs import bf16_to_f64
from .layer import LowpWeight, dequant_weight
from .segments import build_segments


def base_weight(w: LowpWeight) -> np.ndarray:
    """W_d as float64 [N, K]: FP8 codes times the channel scale, or MXFP4 codes times their
    block scale (both products exact in fp64)."""
    Wd, col_scale = dequant_weight(w)
    if col_scale is not None:
        Wd = Wd * col_scale[:, None]
    return Wd


def lora_backward(x_bits, w: LowpWeight, A, B, scale, adapter_id, dy_bits):
    """Returns a dict: ``dx`` float64 [T, K]; ``dA`` list of [K, r_a]; ``dB`` list of
    [r_a, N] (zero for adapters without tokens); ``u`` [T, r_max] and ``t`` [T, r_max] (the
    forward down-projection), zero beyond each token's rank."""
    x = bf16_to_f64(np.asarray(x_bits, dtype=np.uint16))
    dy = bf16_to_f64(np.asarray(dy_bits, dtype=np.uint16))
    n_ad = len(A)
    seg_indptr, sorted_tok = build_segments(adapter_id, n_ad)
    Wd = base_weight(w)                                  # [N, K]
    T, K = x.shape
    r_max = max(int(np.asarray(a).shape[1]) for a in A)
    dx = dy @ Wd                                         # dY . W_d^T, W stored [N, K]
    u = np.zeros((T, r_max))
    t = np.zeros((T, r_max))
    dA, dB = [], []
    for a in range(n_ad):
        Aa = bf16_to_f64(np.asarray(A[a], dtype=np.uint16))     # [K, r]
        Ba = bf16_to_f64(np.asarray(B[a], dtype=np.uint16))     # [r, N]
        r = Aa.shape[1]
        s = float(np.float32(scale[a]))
        R = np.asarray(sorted_tok[seg_indptr[a]:seg_indptr[a + 1]], dtype=np.int64)
        if R.size == 0:
            dA.append(np.zeros((K, r)))
            dB.append(np.zeros((r, Ba.shape[1])))
            continue
        ua = dy[R] @ Ba.T                                # [|R|, r]
        ta = x[R] @ Aa                                   # [|R|, r]
        u[R, :r] = ua
        t[R, :r] = ta
        dx[R] += s * (ua @ Aa.T)
        dA.append(s * (x[R].T @ ua))
        dB.append(s * (ta.T @ dy[R]))
    return {"dx": dx, "dA": dA, "dB": dB, "u": u, "t": t, "seg_indptr": seg_indptr, "sorted_tok": sorted_tok}
