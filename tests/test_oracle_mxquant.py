"""Pins for oracle/mxquant.py.

A second, independent formulation of the MXFP8 rule works on the bf16 bit fields
with integer arithmetic and a brute-force nearest-value search; the two must agree
bit for bit on every bf16 pattern.  Properties of the rule (block maximum lands in
[256, 448] * 2^E unless the scale clamps; round-off within half a grid step) are
checked as well."""

import numpy as np

from oracle import codecs, mxquant

TABLE = codecs.decode_e4m3fn(np.arange(0x7F, dtype=np.uint8))


def _bitfield_quantise(x_bits):
    """Formulation 2: integer bit fields of bf16, exact rationals via float64 ldexp."""
    b = np.asarray(x_bits, dtype=np.uint16).astype(np.int64)
    T, K = b.shape
    blk = b.reshape(T, K // 32, 32)
    mag = blk & 0x7FFF                       # |x| as bits: monotone in |x| for finite x
    ef = (mag.max(axis=2) >> 7) & 0xFF       # biased exponent field of the block maximum
    code = np.maximum(ef - 8, 0)             # floor(log2 m) - 8 + 127, clamped at 0
    e = (blk >> 7) & 0xFF
    m = blk & 0x7F
    sig = np.where(e == 0, m, 128 + m)
    ex = np.where(e == 0, -133, e - 134)     # value = sig * 2^ex
    v = np.ldexp(sig.astype(np.float64), (ex + 127 - code[..., None]).astype(np.int32))
    v = np.minimum(v, 448.0)
    d = np.abs(v.reshape(-1)[:, None] - TABLE[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    codes = np.arange(0x7F)
    even = np.where(cand & (codes % 2 == 0), codes, 999).min(axis=1)
    pick = np.where(cand.sum(axis=1) == 1, np.argmax(cand, axis=1), even)
    q = pick | np.where(((blk >> 15) & 1).reshape(-1) == 1, 0x80, 0)
    return q.reshape(T, K).astype(np.uint8), code.astype(np.uint8)


def _all_finite_bf16():
    bits = np.arange(65536, dtype=np.uint16)
    fin = ((bits >> 7) & 0xFF) != 0xFF
    return bits[fin]


def test_all_bf16_patterns_two_formulations():
    bits = _all_finite_bf16()
    rng = np.random.default_rng(0)
    # every pattern appears, in blocks whose maxima span the whole exponent range
    perm = rng.permutation(bits)
    n = (perm.size // 32) * 32
    x = perm[:n].reshape(-1, 32 * 8)[:, :]  # rows of 8 blocks
    # chunk through to keep the brute-force table search small
    for s in range(0, x.shape[0], 32):
        xs = x[s:s + 32]
        q1, e1 = mxquant.quantize_mxfp8(xs)
        q2, e2 = _bitfield_quantise(xs)
        assert np.array_equal(e1, e2)
        assert np.array_equal(q1, q2)


def test_every_pattern_as_block_maximum():
    # each finite bf16 value once as the maximum of an otherwise small block
    bits = _all_finite_bf16()
    rng = np.random.default_rng(1)
    rows = []
    for b in bits[::7]:
        blk = np.full(32, 0x3C00, np.uint16)           # 2^-7 fillers
        blk[rng.integers(0, 32)] = b
        rows.append(blk)
    x = np.array(rows, np.uint16).reshape(-1, 32)
    q1, e1 = mxquant.quantize_mxfp8(x)
    q2, e2 = _bitfield_quantise(x)
    assert np.array_equal(e1, e2) and np.array_equal(q1, q2)


def test_special_blocks():
    z = np.zeros((1, 32), np.uint16)
    q, e = mxquant.quantize_mxfp8(z)
    assert e[0, 0] == 0 and (q == 0).all()
    negz = np.full((1, 32), 0x8000, np.uint16)
    q, e = mxquant.quantize_mxfp8(negz)
    assert e[0, 0] == 0 and (q == 0x80).all()
    # 1.0 everywhere: E = -8, codes = 256 = 0x78
    one = np.full((1, 32), 0x3F80, np.uint16)
    q, e = mxquant.quantize_mxfp8(one)
    assert e[0, 0] == 127 - 8 and (codecs.decode_e4m3fn(q) == 256.0).all()
    # largest bf16 magnitude: floor(log2) = 127 -> code 246
    big = np.full((1, 32), 0x7F7F, np.uint16)
    q, e = mxquant.quantize_mxfp8(big)
    assert e[0, 0] == 246


def test_properties_on_random_blocks():
    rng = np.random.default_rng(2)
    x32 = (rng.standard_normal((64, 1024)) * np.exp2(rng.integers(-20, 20, (64, 1)))).astype(np.float32)
    bits = (x32.view(np.uint32) >> 16).astype(np.uint16)
    q, e = mxquant.quantize_mxfp8(bits)
    x = codecs.bf16_to_f64(bits).reshape(64, 32, 32)
    dq = mxquant.dequantize_mxfp8(q, e).reshape(64, 32, 32)
    E = e.astype(np.int64) - 127
    m = np.abs(dq).max(axis=2)
    assert (m >= 256 * np.exp2(E) * (1 - 1e-12)).all() and (m <= 448 * np.exp2(E)).all()
    # error: at most half a grid step of the element's binade (grid step <= 2^(E-9+...))
    step = np.exp2(np.floor(np.log2(np.maximum(np.abs(x), 1e-300))) - 3)
    step = np.maximum(step, np.exp2(E - 9)[..., None])
    unsat = np.abs(x) * np.exp2(-E)[..., None] <= 448
    assert (np.abs(dq - x)[unsat] <= step[unsat] / 2 + 1e-300).all()
