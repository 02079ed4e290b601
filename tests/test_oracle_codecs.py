"""Pins for oracle/codecs.py: exhaustive code tables against torch's float8 dtypes
(library routines), the OCP format constants, and an independent nearest-value
encoder."""

import numpy as np
import pytest
import torch

from oracle import codecs


def test_e4m3fn_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = codecs.decode_e4m3fn(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    # sign of zero
    assert np.signbit(ours[0x80]) and not np.signbit(ours[0x00])


def test_e4m3fn_spec_constants():
    d = codecs.decode_e4m3fn
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0
    assert d(0x01) == 2.0 ** -9            # smallest subnormal
    assert d(0x07) == 7 * 2.0 ** -9        # largest subnormal
    assert d(0x08) == 2.0 ** -6            # smallest normal
    assert d(0x38) == 1.0
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    assert np.isfinite(codecs.decode_e4m3fn(np.arange(0x7F, dtype=np.uint8))).all()


def test_e2m1_decode_spec_set():
    vals = codecs.decode_e2m1(np.arange(16))
    assert list(vals[:8]) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(vals[8:]) == [-0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    assert np.signbit(vals[8])


def test_e8m0_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = codecs.decode_e8m0(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert np.array_equal(ours[:255], ref[:255])
    assert ours[127] == 1.0 and ours[0] == 2.0 ** -127


def test_bf16_widen():
    bits = np.arange(65536, dtype=np.uint16)
    ours = codecs.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def _nearest_even_table(values):
    """Independent e4m3fn encoder: brute-force nearest finite value; ties go to the
    code with an even mantissa (even code)."""
    table = codecs.decode_e4m3fn(np.arange(0x7F, dtype=np.uint8))
    a = np.abs(values)
    d = np.abs(a[:, None] - table[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    codes = np.arange(0x7F)
    # among tied candidates take the even code
    pick = np.where(cand & (codes[None, :] % 2 == 0), codes[None, :], 10**6).min(axis=1)
    single = cand.sum(axis=1) == 1
    pick = np.where(single, np.argmax(cand, axis=1), pick)
    return (pick | np.where(np.signbit(values), 0x80, 0)).astype(np.uint8)


def test_e4m3fn_encode_roundtrip_and_ties():
    table = codecs.decode_e4m3fn(np.arange(0x7F, dtype=np.uint8))
    mids = (table[1:] + table[:-1]) / 2
    quarter = table[:-1] + (table[1:] - table[:-1]) / 4
    vals = np.concatenate([table, -table, mids, -mids, quarter, -quarter, [0.0, -0.0]])
    ours = codecs.encode_e4m3fn_rne(vals)
    assert np.array_equal(ours, _nearest_even_table(vals))
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    assert np.array_equal(codecs.decode_e4m3fn(ours[: 127]), table)


def test_e4m3fn_encode_random():
    rng = np.random.default_rng(5)
    v = rng.standard_normal(20000) * np.exp2(rng.integers(-14, 9, 20000))
    v = np.clip(v, -448, 448)
    ours = codecs.encode_e4m3fn_rne(v)
    assert np.array_equal(ours, _nearest_even_table(v))
    assert np.array_equal(ours, torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy())


def test_e4m3fn_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        codecs.encode_e4m3fn_rne(np.array([449.0]))
    with pytest.raises(ValueError):
        codecs.encode_e4m3fn_rne(np.array([np.nan]))
