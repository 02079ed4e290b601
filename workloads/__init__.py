"""Seeded synthetic inputs for the multi-tenant LoRA layer.

This module only draws inputs; it holds none of the layer's arithmetic.  Both the
oracle-based tests and the GPU path consume what it returns.  The base weight is
prepared here the way a serving engine prepares it offline (FP8 per-channel or
MXFP4 quantisation of a float weight); those codes are inputs to the layer.

Five named workloads have the shapes and value distributions of the layer the
pages discuss (sizes in tokens T, reduction K, outputs N):

* ``tiny``          T=4,    K=256,   N=256,   FP8,   2 adapters r=8,   ids [0,1,1,0]
* ``decode_qkv``    T=16,   K=4096,  N=6144,  FP8,   1 adapter  r=16 (all tokens on it)
* ``decode_gateup`` T=64,   K=4096,  N=28672, FP8,   32 adapters r=16, Zipf(1.1) ids
* ``prefill``       T=4096, K=4096,  N=4096,  FP8,   8 adapters r=64, contiguous segments
* ``downproj_fp4``  T=128,  K=21504, N=5376,  MXFP4, 128 adapters r in {8,16,32,64},
                    one token per adapter in random order, s = 16 / r

Distributions: x ~ N(0, 1); W ~ N(0, 0.02) before quantisation; A ~ N(0, sigma_A)
with sigma_A = 1/16 for ``tiny``, 1/64 for K = 4096 and 1/sqrt(21504) for
``downproj_fp4``; B ~ N(0, 0.01).  All sigmas are standard deviations.  bf16 values
are float32 draws rounded to nearest even.  Draw order: ids / segment cuts / ranks,
then x, W, A (adapter by adapter), B.  Seeds: 1001..1005 in the order above.

These stand in for real model weights and for request traces of the popularity
classes Identical (one adapter), Skewed (Zipf), Uniform contiguous segments and
Distinct (one adapter per request); no dataset or checkpoint is used.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "make", "make_custom", "grad_output", "bf16_bits", "bf16_to_f32"]


@dataclass
class Workload:
    name: str
    T: int
    K: int
    N: int
    fmt: str                      # "fp8" or "mxfp4"
    x: np.ndarray                 # uint16 [T, K] bf16 bits
    w_q: np.ndarray               # uint8 [N, K] (fp8) or [N, K/2] (mxfp4)
    w_scale: np.ndarray           # float32 [N] (fp8) or uint8 [N, K/32] (mxfp4)
    A: list                       # uint16 [K, r_a] per adapter
    B: list                       # uint16 [r_a, N] per adapter
    ranks: np.ndarray             # int32 [n_adapters]
    scale: np.ndarray             # float32 [n_adapters]
    ids: np.ndarray               # int32 [T]
    seed: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def n_adapters(self) -> int:
        return len(self.A)

    @property
    def r_max(self) -> int:
        return int(self.ranks.max())


def bf16_bits(x_f32: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    b = np.ascontiguousarray(x_f32, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng, shape, std) -> np.ndarray:
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def quantize_fp8_per_channel(w: np.ndarray):
    """Offline FP8 weight preparation: s[n] = max_k |W[n,k]| / 448, codes = RNE(W / s).

    ``w`` float32 [N, K].  A zero row gets scale 1.  Encoding uses torch's
    float8_e4m3fn conversion (round to nearest even) after clamping to +-448.
    """
    amax = np.abs(w).max(axis=1)
    s = (amax / np.float32(448.0)).astype(np.float32)
    s[s == 0] = np.float32(1.0)
    v = np.clip(w / s[:, None], -448.0, 448.0).astype(np.float32)
    q = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return q, s


_E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
_E2M1_MID = (_E2M1_GRID[1:] + _E2M1_GRID[:-1]) / 2


def quantize_mxfp4(w: np.ndarray):
    """Offline MXFP4 weight preparation (OCP MX v1.0 style, blocks of 32 along K).

    Per block: E = floor(log2 amax) - 2 (2 = largest e2m1 exponent), scale code
    E + 127 clamped to [0, 254] (an all-zero block gets code 0); elements are
    w / 2^E rounded to the nearest e2m1 value, ties to the even code, saturating
    at 6.  Element k of row n goes to the low nibble of byte k//2 when k is even.
    Returns ``(packed uint8 [N, K/2], scales uint8 [N, K/32])``.
    """
    N, K = w.shape
    wb = w.astype(np.float64).reshape(N, K // 32, 32)
    amax = np.abs(wb).max(axis=2)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))
    E = np.where(amax > 0, e.astype(np.int64) - 1 - 2, -127)
    code = np.clip(E + 127, 0, 254)
    E = code - 127
    v = np.ldexp(wb, (-E)[..., None].astype(np.int32))
    a = np.abs(v)
    idx = np.searchsorted(_E2M1_MID, a, side="left")
    tie = (idx < 7) & (a == _E2M1_MID[np.minimum(idx, 6)])
    idx = np.where(tie & (idx % 2 == 1), idx + 1, idx)
    nib = (idx | np.where(np.signbit(v), 8, 0)).astype(np.uint8).reshape(N, K)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return packed, code.astype(np.uint8)


def _zipf_ids(rng, T, n, s):
    p = np.arange(1, n + 1, dtype=np.float64) ** (-s)
    p /= p.sum()
    return rng.choice(n, size=T, p=p).astype(np.int32)


def _contiguous_ids(rng, T, n):
    cuts = np.sort(rng.choice(np.arange(1, T), size=n - 1, replace=False))
    lengths = np.diff(np.concatenate([[0], cuts, [T]]))
    return np.repeat(np.arange(n, dtype=np.int32), lengths)


def make_custom(T, K, N, fmt, ranks, ids, scale, seed, *, name="custom", x_std=1.0,
                w_std=0.02, a_std=None, b_std=0.01, zero_w=False, zero_b=False) -> Workload:
    """Draw x, W, A, B for the given shape, adapters and ids (ids/ranks already chosen)."""
    rng = np.random.default_rng(seed)
    return _draw(rng, name, T, K, N, fmt, np.asarray(ranks, np.int32), np.asarray(ids, np.int32),
                 np.asarray(scale, np.float32), seed, x_std, w_std,
                 a_std if a_std is not None else 1.0 / np.sqrt(K), b_std, zero_w, zero_b)


def _draw(rng, name, T, K, N, fmt, ranks, ids, scale, seed, x_std, w_std, a_std, b_std,
          zero_w=False, zero_b=False) -> Workload:
    x = bf16_bits(_normal(rng, (T, K), x_std))
    w = _normal(rng, (N, K), w_std)
    if zero_w:
        w[:] = 0
    if fmt == "fp8":
        w_q, w_s = quantize_fp8_per_channel(w)
    elif fmt == "mxfp4":
        w_q, w_s = quantize_mxfp4(w)
    else:
        raise ValueError(fmt)
    del w
    A = [bf16_bits(_normal(rng, (K, int(r)), a_std)) for r in ranks]
    B = [bf16_bits(_normal(rng, (int(r), N), b_std)) for r in ranks]
    if zero_b:
        B = [np.zeros_like(b) for b in B]
    return Workload(name, T, K, N, fmt, x, w_q, w_s, A, B, ranks, scale, ids, seed)


def grad_output(T: int, N: int, seed: int, std: float = 1.0) -> np.ndarray:
    """A seeded gradient dY of a loss with respect to the layer output, bf16 bits [T, N],
    drawn N(0, std) (the backward's input besides the forward's)."""
    rng = np.random.default_rng(seed)
    return bf16_bits(_normal(rng, (T, N), std))


WORKLOADS = {
    "tiny": dict(T=4, K=256, N=256, fmt="fp8", seed=1001),
    "decode_qkv": dict(T=16, K=4096, N=6144, fmt="fp8", seed=1002),
    "decode_gateup": dict(T=64, K=4096, N=28672, fmt="fp8", seed=1003),
    "prefill": dict(T=4096, K=4096, N=4096, fmt="fp8", seed=1004),
    "downproj_fp4": dict(T=128, K=21504, N=5376, fmt="mxfp4", seed=1005),
}


def make(name: str, seed: int | None = None) -> Workload:
    """Build one of the named workloads (seeded; identical on every machine)."""
    cfg = WORKLOADS[name]
    seed = cfg["seed"] if seed is None else seed
    rng = np.random.default_rng(seed)
    T, K, N, fmt = cfg["T"], cfg["K"], cfg["N"], cfg["fmt"]
    if name == "tiny":
        n, ranks, ids = 2, np.full(2, 8, np.int32), np.array([0, 1, 1, 0], np.int32)
        scale, a_std = np.full(n, 2.0, np.float32), 1.0 / 16
    elif name == "decode_qkv":
        n, ranks, ids = 1, np.full(1, 16, np.int32), np.zeros(T, np.int32)
        scale, a_std = np.full(n, 2.0, np.float32), 1.0 / 64
    elif name == "decode_gateup":
        n = 32
        ids = _zipf_ids(rng, T, n, 1.1)
        ranks, scale, a_std = np.full(n, 16, np.int32), np.full(n, 2.0, np.float32), 1.0 / 64
    elif name == "prefill":
        n = 8
        ids = _contiguous_ids(rng, T, n)
        ranks, scale, a_std = np.full(n, 64, np.int32), np.full(n, 1.0, np.float32), 1.0 / 64
    elif name == "downproj_fp4":
        n = 128
        ranks = rng.choice(np.array([8, 16, 32, 64], np.int32), size=n)
        ids = rng.permutation(n).astype(np.int32)
        scale, a_std = (16.0 / ranks).astype(np.float32), 1.0 / np.sqrt(K)
    else:
        raise KeyError(name)
    wl = _draw(rng, name, T, K, N, fmt, ranks, ids, scale, seed, 1.0, 0.02, a_std, 0.01)
    return wl
