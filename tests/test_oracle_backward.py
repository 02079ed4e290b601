"""Pins for oracle/backward.py, independent of its formulas:

* dX equals dY times the transposed merged weight W_d + s_a A_a B_a, built per adapter
  ("Punica" README, Overview: x@(W + A@B) = x@W + x@A@B);
* the forward oracle (layer.layer, act="bf16") is linear in x, in A_a and in B_a separately,
  so the loss L = sum_t <dY[t], y[t]> changes by exactly delta * (the gradient's element) when
  one element of x, A_a or B_a changes by delta -- checked element by element;
* exact rational brute force (fractions.Fraction) of every gradient on a tiny batch;
* special cases: B = 0 gives dA = 0 and dX = dY W_d^T; dY = 0 gives zeros; gradients of
  adapters without tokens are zero.
"""

from fractions import Fraction

import numpy as np

import workloads
from oracle import backward as BW
from oracle.codecs import bf16_to_f64
from oracle.layer import LowpWeight, layer


def _case(T=6, K=64, N=32, fmt="fp8", ranks=(4, 8, 3), seed=1, ids=None):
    rng = np.random.default_rng(seed)
    if ids is None:
        ids = rng.integers(0, len(ranks), T)
    wl = workloads.make_custom(T, K, N, fmt, list(ranks), ids, [1.5, 0.5, 2.0][:len(ranks)], seed, a_std=0.2,
                               b_std=0.1)
    dy = workloads.bf16_bits(rng.standard_normal((T, N)).astype(np.float32))
    return wl, dy


def _w(wl):
    return LowpWeight(wl.fmt, wl.w_q, wl.w_scale)


def test_dx_is_dy_times_the_merged_weight():
    for fmt in ("fp8", "mxfp4"):
        wl, dy = _case(T=9, K=128, N=64, fmt=fmt, seed=3)
        g = BW.lora_backward(wl.x, _w(wl), wl.A, wl.B, wl.scale, wl.ids, dy)
        Wd = BW.base_weight(_w(wl))                       # [N, K]
        dyf = bf16_to_f64(dy)
        for t in range(wl.T):
            a = wl.ids[t]
            merged = Wd.T + float(np.float32(wl.scale[a])) * (bf16_to_f64(wl.A[a]) @ bf16_to_f64(wl.B[a]))  # [K, N]
            np.testing.assert_allclose(g["dx"][t], merged @ dyf[t], rtol=1e-12, atol=1e-12)


def _loss(wl, dy, x=None, A=None, B=None):
    y = layer(wl.x if x is None else x, _w(wl), wl.A if A is None else A, wl.B if B is None else B, wl.scale, wl.ids,
              act="bf16")["y"]
    return float(np.sum(bf16_to_f64(dy) * y))


def test_gradients_are_the_forward_oracles_linear_responses():
    wl, dy = _case(T=7, K=64, N=32, seed=5)
    g = BW.lora_backward(wl.x, _w(wl), wl.A, wl.B, wl.scale, wl.ids, dy)
    L0 = _loss(wl, dy)
    rng = np.random.default_rng(9)
    newval = workloads.bf16_bits(np.array([0.75], np.float32))[0]       # a bf16 value to move to
    for _ in range(12):                                                 # x elements
        t, k = int(rng.integers(wl.T)), int(rng.integers(wl.K))
        x = wl.x.copy()
        x[t, k] = newval
        d = float(bf16_to_f64(np.array([newval], np.uint16))[0] - bf16_to_f64(wl.x[t:t + 1, k])[0])
        assert abs((_loss(wl, dy, x=x) - L0) - d * g["dx"][t, k]) <= 1e-9 * max(1.0, abs(L0))
    for a in range(wl.n_adapters):
        if not np.any(wl.ids == a):
            continue
        for _ in range(6):                                              # A_a and B_a elements
            A = [m.copy() for m in wl.A]
            k, j = int(rng.integers(wl.K)), int(rng.integers(A[a].shape[1]))
            d = 0.75 - float(bf16_to_f64(A[a][k:k + 1, j])[0])
            A[a][k, j] = newval
            assert abs((_loss(wl, dy, A=A) - L0) - d * g["dA"][a][k, j]) <= 1e-9 * max(1.0, abs(L0))
            B = [m.copy() for m in wl.B]
            j, n = int(rng.integers(B[a].shape[0])), int(rng.integers(wl.N))
            d = 0.75 - float(bf16_to_f64(B[a][j:j + 1, n])[0])
            B[a][j, n] = newval
            assert abs((_loss(wl, dy, B=B) - L0) - d * g["dB"][a][j, n]) <= 1e-9 * max(1.0, abs(L0))


def test_exact_rationals_on_a_tiny_batch():
    wl, dy = _case(T=3, K=32, N=16, ranks=(2, 3), seed=11, ids=np.array([1, 0, 1]))
    g = BW.lora_backward(wl.x, _w(wl), wl.A, wl.B, wl.scale, wl.ids, dy)
    F = lambda v: Fraction(float(v))  # noqa: E731  (every value involved is a float exactly)
    x = bf16_to_f64(wl.x)
    d = bf16_to_f64(dy)
    Wd = BW.base_weight(_w(wl))
    for t in range(wl.T):
        a = int(wl.ids[t])
        A, B, s = bf16_to_f64(wl.A[a]), bf16_to_f64(wl.B[a]), F(np.float32(wl.scale[a]))
        r = A.shape[1]
        u = [sum(F(d[t, n]) * F(B[j, n]) for n in range(wl.N)) for j in range(r)]
        for k in range(wl.K):
            ex = sum(F(d[t, n]) * F(Wd[n, k]) for n in range(wl.N)) + s * sum(u[j] * F(A[k, j]) for j in range(r))
            assert abs(float(ex) - g["dx"][t, k]) <= 1e-14 * max(1.0, abs(float(ex)))
    for a in range(wl.n_adapters):
        A, B, s = bf16_to_f64(wl.A[a]), bf16_to_f64(wl.B[a]), F(np.float32(wl.scale[a]))
        R = [t for t in range(wl.T) if wl.ids[t] == a]
        r = A.shape[1]
        for k in range(wl.K):
            for j in range(r):
                ex = s * sum(F(x[t, k]) * sum(F(d[t, n]) * F(B[j, n]) for n in range(wl.N)) for t in R)
                assert abs(float(ex) - g["dA"][a][k, j]) <= 1e-14 * max(1.0, abs(float(ex)))
        for j in range(r):
            for n in range(wl.N):
                ex = s * sum(sum(F(x[t, k]) * F(A[k, j]) for k in range(wl.K)) * F(d[t, n]) for t in R)
                assert abs(float(ex) - g["dB"][a][j, n]) <= 1e-14 * max(1.0, abs(float(ex)))


def test_special_cases():
    wl, dy = _case(T=8, K=64, N=32, ranks=(4, 8, 3), seed=13, ids=np.array([0, 0, 1, 1, 0, 1, 1, 0]))
    Wd = BW.base_weight(_w(wl))
    zb = [np.zeros_like(b) for b in wl.B]
    g = BW.lora_backward(wl.x, _w(wl), wl.A, zb, wl.scale, wl.ids, dy)
    assert all(not m.any() for m in g["dA"]) and not g["u"].any()
    np.testing.assert_array_equal(g["dx"], bf16_to_f64(dy) @ Wd)
    g = BW.lora_backward(wl.x, _w(wl), wl.A, wl.B, wl.scale, wl.ids, np.zeros_like(dy))
    assert not g["dx"].any() and all(not m.any() for m in g["dA"] + g["dB"])
    g = BW.lora_backward(wl.x, _w(wl), wl.A, wl.B, wl.scale, wl.ids, dy)
    assert not g["dA"][2].any() and not g["dB"][2].any()          # adapter 2 has no tokens
    assert g["dA"][0].any() and g["dB"][1].any()
