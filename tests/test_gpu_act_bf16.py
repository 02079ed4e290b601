"""GPU parity of the 16-bit activation variant (LORA_ACT_BF16): the base product reads
the bf16 x as it is, W widened to bf16, bf16 MFMA.  Compared with the oracle's
act="bf16" layer to the same bars as the MXFP8 path; the output's offset from the
MXFP8 oracle must match the difference of the two oracles, so that a path that still
quantised x would fail.
Cases: the 16-token qkv workload at full size (fused, unfused, base only, segments
built in the launch); the 64-token gate-up and the 4096-token prefill workloads (64 x 128
tiles, prefill on sampled rows); 16-token batches at the gate-up and MXFP4 down-projection
shapes; ragged, tiny and many-adapter shapes in both formats, on 64 x 128 tiles and, where
N % 128 != 0, on 16-token stream tiles with column-tile counts of 6 and 10 (the XCD
grouping with and without a tail); past 128 tokens with FP8 and N % 256 == 0, the
down-projection pre-pass and 64 x 256 tiles (one row past a tile, a ragged last tile,
segments built by the call)."""

import numpy as np
import pytest

import workloads
from gpu_util import assert_t_close, assert_y_close, errors, named, run_gpu, run_oracle, sample_rows

pytestmark = pytest.mark.gpu


def _check(wl, g, what, base_only=False, rows=None):
    ref = run_oracle(wl, rows, act="bf16")
    key = "y_base" if base_only else "y"
    sel = slice(None) if rows is None else np.asarray(rows)
    y = g["y"][sel]
    m, f = assert_y_close(y, ref[key], what)
    if not base_only:
        assert_t_close(g["t"][sel].astype(np.float64), ref["t"], what)
    # x was not quantised: with d = (bf16 oracle) - (MXFP8 oracle), the output's offset
    # from the MXFP8 oracle projects onto d with coefficient ~1 (~0 if x were quantised);
    # the bf16 rounding of y is uncorrelated with d
    y8 = run_oracle(wl, rows)[key]
    d = ref[key] - y8
    c = float(np.vdot(y - y8, d) / np.vdot(d, d))
    _, f8 = errors(y, y8)
    assert 0.8 < c < 1.2, f"{what}: projection on the activation-quantisation difference {c:.3f}"
    print(f"  y max_rel={m:.2e} frob={f:.2e} (MXFP8 oracle: frob={f8:.2e}; projection {c:.3f})", flush=True)


@pytest.mark.parametrize("mode", ["fused", "unfused", "base_only", "build"])
def test_decode_qkv_bf16_activations(mode):
    print(f"[case] act_bf16 decode_qkv {mode}", flush=True)
    wl = named("decode_qkv")
    g = run_gpu(wl, fused=(mode != "unfused"), base_only=(mode == "base_only"), build=(mode == "build"),
                act_bf16=True)
    assert g["status"] == 0 and g["err"] == 0
    _check(wl, g, f"decode_qkv {mode}", base_only=(mode == "base_only"))


@pytest.mark.parametrize("name,build", [("decode_gateup", False), ("decode_gateup", True), ("prefill", False)])
def test_multi_tile_workloads_bf16_activations(name, build):
    print(f"[case] act_bf16 {name} build={build}", flush=True)
    wl = named(name)
    rows = None
    if name == "prefill":  # 96 random rows plus the first and last row of every segment
        rows = sample_rows(wl, 96, 9)
        assert 0 in rows
    g = run_gpu(wl, fused=True, build=build, act_bf16=True)
    assert g["status"] == 0 and g["err"] == 0
    _check(wl, g, f"{name} build={build}", rows=rows)


CASES = [
    # T, K, N, fmt, ranks, seed
    (16, 4096, 28672, "fp8", [16] * 32, 41),              # gate-up shape, 16 tokens
    (16, 21504, 5376, "mxfp4", [8, 16, 32, 64] * 4, 42),  # MXFP4 down-projection shape
    (1, 128, 64, "fp8", [8], 43),
    (5, 256, 128, "mxfp4", [16, 8], 44),
    (13, 1152, 320, "fp8", [8, 24, 64], 45),
    (16, 640, 192, "mxfp4", [32, 16], 46),
    (17, 512, 192, "fp8", [8, 16, 24, 32], 47),           # stream tiles, 6 column tiles: plain order only
    (37, 384, 256, "mxfp4", [64, 40, 8], 48),             # 64 x 128 tiles, ragged
    (130, 1024, 320, "fp8", [16, 64] * 32, 49),           # stream tiles, 10 column tiles (8 + a tail of 2)
    (300, 768, 256, "fp8", [48, 8, 16, 64], 50),          # down-projection items of 64 tokens
    (200, 4096, 256, "mxfp4", [64, 8, 32, 16, 48] * 14, 51),
    # past 128 tokens, FP8, N % 256 == 0: the rows pre-pass then 64 x 256 tiles
    (129, 640, 512, "fp8", [8, 64, 24], 53),              # one row past two token tiles
    (1000, 1152, 768, "fp8", [16, 32] * 20, 54),          # 3 column blocks, 16 token tiles (last ragged)
]


@pytest.mark.parametrize("case", CASES, ids=[f"T{c[0]}_K{c[1]}_N{c[2]}_{c[3]}_a{len(c[4])}" for c in CASES])
@pytest.mark.parametrize("fused", [True, False], ids=["fused", "unfused"])
def test_shapes_bf16_activations(case, fused):
    T, K, N, fmt, ranks, seed = case
    print(f"[case] act_bf16 {case} fused={fused}", flush=True)
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, len(ranks), T)
    wl = workloads.make_custom(T, K, N, fmt, ranks, ids, [2.0] * len(ranks), seed, a_std=0.1, b_std=0.05)
    g = run_gpu(wl, fused=fused, act_bf16=True)
    assert g["status"] == 0
    _check(wl, g, str(case))


@pytest.mark.parametrize("N", [384, 512], ids=["tiles_64x128", "tiles_64x256"])
def test_bf16_activations_deterministic_and_segments_built(N):
    print(f"[case] act_bf16 T=300 N={N} build, determinism", flush=True)
    rng = np.random.default_rng(52)
    ids = rng.integers(0, 6, 300)
    wl = workloads.make_custom(300, 1024, N, "fp8", [8, 16, 32, 64, 16, 8], ids, [1.0] * 6, 52,
                               a_std=0.1, b_std=0.05)
    g1 = run_gpu(wl, fused=True, build=True, act_bf16=True)
    g2 = run_gpu(wl, fused=True, act_bf16=True)
    assert g1["status"] == 0 and g1["err"] == 0
    assert np.array_equal(g1["y_bits"], g2["y_bits"])
    _check(wl, g1, f"T300 N={N} build")
