"""Pins for oracle/layer.py.

* a hand-worked example (tests/golden/handworked_fp8_two_adapters.json);
* exact rational brute force (fractions.Fraction) on the tiny workload, FP8 and MXFP4;
* the merged-weight identity x.(W + s A B) = x.W + s (x.A).B, per token, on inputs whose
  MXFP8 form is exact (Punica README: y = x@(W + A@B) = x@W + x@A@B);
* zero-B gives exactly the base GEMM, zero-W gives exactly the adapter term;
* invariance under token permutation and adapter relabelling;
* one adapter reduces to plain numpy matmuls;
* the exactness guard's fallback on a wide dynamic range;
* the 16-bit activation variant (act="bf16"): exact rational brute force, the
  merged-weight identity on x that is not MXFP8-exact, bitwise equality with the
  MXFP8 form where that form is exact, and its guard fallback.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import workloads
from oracle import codecs, layer as L
from oracle.layer import LowpWeight

HERE = os.path.dirname(__file__)


def _weight(wl):
    return LowpWeight(wl.fmt, wl.w_q, wl.w_scale)


def test_golden_handworked():
    g = json.load(open(os.path.join(HERE, "golden", "handworked_fp8_two_adapters.json")))
    K, N = g["K"], g["N"]
    x = np.zeros((2, K), np.float32)
    for t, k, v in g["x_nonzero"]:
        x[t, k] = v
    wq = np.zeros((N, K), np.uint8)
    for n, k, c in g["w_codes_nonzero"]:
        if k == "all":
            wq[n, :] = c
        else:
            wq[n, k] = c
    A, B = [], []
    for spec, b in zip(g["A"], g["B"]):
        a = np.zeros((K, spec["rank"]), np.float32)
        for k, j, v in spec["nonzero"]:
            a[k, j] = v
        A.append(workloads.bf16_bits(a))
        B.append(workloads.bf16_bits(np.array(b, np.float32)))
    out = L.layer(workloads.bf16_bits(x), LowpWeight("fp8", wq, np.array(g["w_scale"], np.float32)),
                  A, B, np.array(g["s"], np.float32), g["ids"])
    e = g["expect"]
    assert out["x_sc"].tolist() == e["x_sc"]
    xq = np.zeros((2, K), np.uint8)
    for t, k, c in e["x_q_nonzero"]:
        xq[t, k] = c
    assert np.array_equal(out["x_q"], xq)
    assert out["y_base"].tolist() == e["y_base"]
    assert out["t"].tolist() == e["t"]
    assert out["y"].tolist() == e["y"]
    assert out["seg_indptr"].tolist() == e["seg_indptr"]
    assert out["sorted_tok"].tolist() == e["sorted_tok"]


def _exact_layer(wl, act="mxfp8"):
    """Exact rationals: base sum, channel scale, adapter terms (slow; tiny shapes only).

    act="bf16": the base sum reads the bf16 x itself (the 16-bit activation variant)."""
    from oracle.mxquant import quantize_mxfp8, dequantize_mxfp8
    xb = codecs.bf16_to_f64(wl.x)
    X = dequantize_mxfp8(*quantize_mxfp8(wl.x)) if act == "mxfp8" else xb
    Wd, cs = L.dequant_weight(_weight(wl))
    T, N = X.shape[0], Wd.shape[0]
    Xf = [[Fraction(v) for v in row] for row in X]
    Wf = [[Fraction(v) for v in row] for row in Wd]
    y = [[None] * N for _ in range(T)]
    for t in range(T):
        a = int(wl.ids[t])
        Af = [[Fraction(v) for v in row] for row in codecs.bf16_to_f64(wl.A[a])]
        Bf = [[Fraction(v) for v in row] for row in codecs.bf16_to_f64(wl.B[a])]
        r = len(Af[0])
        tt = [sum(Fraction(xb[t, k]) * Af[k][j] for k in range(len(Af))) for j in range(r)]
        s = Fraction(float(np.float32(wl.scale[a])))
        for n in range(N):
            base = sum(Xf[t][k] * Wf[n][k] for k in range(len(Xf[t])))
            if cs is not None:
                base *= Fraction(float(cs[n]))
            y[t][n] = (base, s * sum(tt[j] * Bf[j][n] for j in range(r)))
    return y


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_fraction_brute_force(fmt):
    ranks = np.array([8, 4], np.int32)
    wl = workloads.make_custom(4, 64, 24, fmt, ranks, [0, 1, 1, 0], [2.0, 0.5], seed=11, a_std=1 / 8)
    out = L.layer(wl.x, _weight(wl), wl.A, wl.B, wl.scale, wl.ids)
    ex = _exact_layer(wl)
    for t in range(4):
        for n in range(24):
            base, lora = ex[t][n]
            # base: exact sum, one rounding for the channel scale (FP8) or none (MXFP4)
            assert abs(Fraction(out["y_base"][t, n]) - base) <= abs(base) * Fraction(1, 2 ** 52)
            assert abs(float(lora) - out["y_lora"][t, n]) <= 1e-13 * max(1.0, abs(float(lora)))


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_fraction_brute_force_bf16_activations(fmt):
    ranks = np.array([8, 4], np.int32)
    wl = workloads.make_custom(4, 64, 24, fmt, ranks, [0, 1, 1, 0], [2.0, 0.5], seed=12, a_std=1 / 8)
    out = L.layer(wl.x, _weight(wl), wl.A, wl.B, wl.scale, wl.ids, act="bf16")
    assert out["x_q"] is None and out["x_sc"] is None
    ex = _exact_layer(wl, act="bf16")
    for t in range(4):
        for n in range(24):
            base, lora = ex[t][n]
            assert abs(Fraction(out["y_base"][t, n]) - base) <= abs(base) * Fraction(1, 2 ** 52)
            assert abs(float(lora) - out["y_lora"][t, n]) <= 1e-13 * max(1.0, abs(float(lora)))
    # random bf16 x is not MXFP8-exact: the two activation forms must give different sums
    assert not np.array_equal(out["y_base"], L.layer(wl.x, _weight(wl), wl.A, wl.B, wl.scale, wl.ids)["y_base"])


def test_fraction_brute_force_tiny_workload():
    wl = workloads.make("tiny")
    out = L.layer(wl.x, _weight(wl), wl.A, wl.B, wl.scale, wl.ids)
    ex = _exact_layer(wl)
    for t in range(wl.T):
        for n in range(0, wl.N, 17):
            base, lora = ex[t][n]
            assert abs(Fraction(out["y_base"][t, n]) - base) <= abs(base) * Fraction(1, 2 ** 52)
            assert abs(float(lora) - out["y_lora"][t, n]) <= 1e-13


def _grid_x(rng, T, K):
    """x = k/8 with |k| <= 7: its MXFP8 form is exact (see module docstring)."""
    k = rng.integers(-7, 8, size=(T, K)).astype(np.float32)
    return workloads.bf16_bits(k / 8)


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_merged_weight_identity(fmt):
    rng = np.random.default_rng(21)
    T, K, N, n_ad = 12, 128, 40, 3
    ranks = np.array([4, 16, 8], np.int32)
    ids = rng.integers(0, n_ad, T)
    wl = workloads.make_custom(T, K, N, fmt, ranks, ids, [2.0, 0.5, 1.0], seed=22)
    wl.x = _grid_x(rng, T, K)
    out = L.layer(wl.x, _weight(wl), wl.A, wl.B, wl.scale, wl.ids)
    from oracle.mxquant import quantize_mxfp8, dequantize_mxfp8
    assert np.array_equal(dequantize_mxfp8(*quantize_mxfp8(wl.x)), codecs.bf16_to_f64(wl.x))
    Wd, cs = L.dequant_weight(_weight(wl))
    Wfull = (Wd * (cs[:, None] if cs is not None else 1.0)).T          # [K, N]
    x = codecs.bf16_to_f64(wl.x)
    for t in range(T):
        a = ids[t]
        merged = Wfull + float(wl.scale[a]) * codecs.bf16_to_f64(wl.A[a]) @ codecs.bf16_to_f64(wl.B[a])
        ref = x[t] @ merged
        assert np.allclose(out["y"][t], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_bf16_activations_merged_weight_identity_and_mxfp8_exact_case(fmt):
    rng = np.random.default_rng(23)
    T, K, N, n_ad = 10, 256, 48, 3
    ranks = np.array([8, 4, 16], np.int32)
    ids = rng.integers(0, n_ad, T)
    wl = workloads.make_custom(T, K, N, fmt, ranks, ids, [1.0, 0.5, 2.0], seed=24)
    # (1) arbitrary bf16 x: y = x @ (W + s_a A_a B_a) per token with x as it is
    out = L.layer(wl.x, _weight(wl), wl.A, wl.B, wl.scale, wl.ids, act="bf16")
    Wd, cs = L.dequant_weight(_weight(wl))
    Wfull = (Wd * (cs[:, None] if cs is not None else 1.0)).T
    x = codecs.bf16_to_f64(wl.x)
    for t in range(T):
        a = ids[t]
        merged = Wfull + float(wl.scale[a]) * codecs.bf16_to_f64(wl.A[a]) @ codecs.bf16_to_f64(wl.B[a])
        ref = x[t] @ merged
        assert np.allclose(out["y"][t], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    # (2) x whose MXFP8 form is exact: both activation forms give the same bits
    wl.x = _grid_x(rng, T, K)
    a16 = L.layer(wl.x, _weight(wl), wl.A, wl.B, wl.scale, wl.ids, act="bf16")
    a8 = L.layer(wl.x, _weight(wl), wl.A, wl.B, wl.scale, wl.ids)
    assert np.array_equal(a16["y"], a8["y"]) and np.array_equal(a16["y_base"], a8["y_base"])


def test_bf16_activations_guard_fallback_and_zero_rows():
    # a row with entries 2^120 apart and an all-zero row
    K, N = 64, 5
    x = np.zeros((2, K), np.float32)
    x[0, :32] = 2.0 ** 60 * np.arange(1, 33)
    x[0, 32:] = 2.0 ** -60 * np.arange(1, 33)
    bits = workloads.bf16_bits(x)
    rng = np.random.default_rng(1)
    wq = rng.integers(0, 0x7F, (N, K)).astype(np.uint8) | (rng.integers(0, 2, (N, K)) << 7).astype(np.uint8)
    w = LowpWeight("fp8", wq, np.full(N, 0.5, np.float32))
    y = L.base_gemm_bf16(bits, w)
    xb = codecs.bf16_to_f64(bits)
    Wd = codecs.decode_e4m3fn(wq)
    for n in range(N):
        exact = sum(Fraction(a) * Fraction(b) for a, b in zip(xb[0], Wd[n])) * Fraction(1, 2)
        assert abs(Fraction(y[0, n]) - exact) <= abs(exact) * Fraction(1, 2 ** 53)
    assert not y[1].any()
    with pytest.raises(ValueError):
        L.layer(bits, w, [workloads.bf16_bits(np.zeros((K, 4), np.float32))],
                [workloads.bf16_bits(np.zeros((4, N), np.float32))], np.ones(1, np.float32), [0, 0], act="fp16")


def test_zero_b_is_exactly_base_and_zero_w_is_exactly_lora():
    wl = workloads.make_custom(8, 96, 33, "fp8", [4, 4], [0, 1] * 4, [2.0, 2.0], seed=5, zero_b=True)
    out = L.layer(wl.x, _weight(wl), wl.A, wl.B, wl.scale, wl.ids)
    assert np.array_equal(out["y"], out["y_base"]) and not out["y_lora"].any()
    wl = workloads.make_custom(8, 96, 33, "mxfp4", [4, 4], [0, 1] * 4, [2.0, 2.0], seed=5, zero_w=True)
    out = L.layer(wl.x, _weight(wl), wl.A, wl.B, wl.scale, wl.ids)
    assert not out["y_base"].any() and np.array_equal(out["y"], out["y_lora"])


def test_token_permutation_and_adapter_relabelling():
    rng = np.random.default_rng(8)
    T, n_ad = 30, 5
    ids = rng.integers(0, n_ad, T)
    wl = workloads.make_custom(T, 64, 20, "fp8", [2, 4, 8, 16, 4], ids, [1, 2, 0.5, 0.25, 4], seed=9)
    ref = L.layer(wl.x, _weight(wl), wl.A, wl.B, wl.scale, wl.ids)["y"]
    p = rng.permutation(T)
    y = L.layer(wl.x[p], _weight(wl), wl.A, wl.B, wl.scale, wl.ids[p])["y"]
    assert np.allclose(y, ref[p], rtol=1e-12, atol=1e-14)
    pi = rng.permutation(n_ad)                     # adapter a becomes pi[a]
    inv = np.argsort(pi)
    A2 = [wl.A[inv[b]] for b in range(n_ad)]
    B2 = [wl.B[inv[b]] for b in range(n_ad)]
    s2 = wl.scale[inv]
    y = L.layer(wl.x, _weight(wl), A2, B2, s2, pi[wl.ids])["y"]
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-14)


def test_single_adapter_reduces_to_plain_numpy():
    wl = workloads.make_custom(16, 512, 96, "fp8", [16], np.zeros(16, int), [2.0], seed=3)
    out = L.layer(wl.x, _weight(wl), wl.A, wl.B, wl.scale, wl.ids)
    from oracle.mxquant import quantize_mxfp8, dequantize_mxfp8
    Xd = dequantize_mxfp8(*quantize_mxfp8(wl.x))
    Wd = codecs.decode_e4m3fn(wl.w_q) * wl.w_scale.astype(np.float64)[:, None]
    x = codecs.bf16_to_f64(wl.x)
    ref = Xd @ Wd.T + 2.0 * (x @ codecs.bf16_to_f64(wl.A[0])) @ codecs.bf16_to_f64(wl.B[0])
    assert np.allclose(out["y"], ref, rtol=1e-12, atol=1e-12)


def test_mxfp4_nibble_order_and_scale():
    # row 0: k0 = 0.5 (nibble 1, low), k1 = 1.0 (nibble 2, high), k2 = -6 (0xF low); scale 2^1
    q = np.zeros((1, 16), np.uint8)
    q[0, 0] = 0x21
    q[0, 1] = 0x0F
    sc = np.array([[128]], np.uint8)
    Wd, cs = L.dequant_weight(LowpWeight("mxfp4", q, sc))
    assert cs is None and Wd[0, :3].tolist() == [1.0, 2.0, -12.0] and not Wd[0, 3:].any()


def test_exactness_guard_fallback():
    # two blocks 200 binades apart: the common quantum is tiny, the guard fails, fsum is used
    K, N = 64, 3
    x = np.zeros((1, K), np.float32)
    x[0, :32] = 2.0 ** 60 * np.arange(1, 33)
    x[0, 32:] = 2.0 ** -60 * np.arange(1, 33)
    bits = workloads.bf16_bits(x)
    rng = np.random.default_rng(0)
    wq = rng.integers(0, 0x7F, (N, K)).astype(np.uint8) | (rng.integers(0, 2, (N, K)) << 7).astype(np.uint8)
    w = LowpWeight("fp8", wq, np.ones(N, np.float32))
    from oracle.mxquant import quantize_mxfp8, dequantize_mxfp8
    xq, xs = quantize_mxfp8(bits)
    y = L.base_gemm(xq, xs, w)
    X = dequantize_mxfp8(xq, xs)
    Wd = codecs.decode_e4m3fn(wq)
    for n in range(N):
        exact = sum(Fraction(a) * Fraction(b) for a, b in zip(X[0], Wd[n]))
        assert Fraction(y[0, n]) - exact == 0 or abs(Fraction(y[0, n]) - exact) <= abs(exact) * Fraction(1, 2 ** 53)
