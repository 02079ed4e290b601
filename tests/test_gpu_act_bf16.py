"""GPU parity of the 16-bit activation variant (LORA_ACT_BF16): the base product reads
the bf16 x as it is, W widened to bf16, bf16 MFMA.  Compared with the oracle's
act="bf16" layer to the same bars as the MXFP8 path; the output's offset from the
MXFP8 oracle must match the difference of the two oracles, so that a path that still
quantised x would fail.
Cases: the 16-token qkv workload at full size (fused, unfused, base only, segments
built in the launch), 16-token batches at the gate-up and MXFP4 down-projection shapes,
ragged and tiny shapes in both formats, and the token limit."""

import numpy as np
import pytest

import workloads
from gpu_util import assert_t_close, assert_y_close, errors, named, run_gpu, run_oracle

pytestmark = pytest.mark.gpu


def _check(wl, g, what, base_only=False):
    ref = run_oracle(wl, act="bf16")
    key = "y_base" if base_only else "y"
    m, f = assert_y_close(g["y"], ref[key], what)
    if not base_only:
        assert_t_close(g["t"].astype(np.float64), ref["t"], what)
    # x was not quantised: with d = (bf16 oracle) - (MXFP8 oracle), the output's offset
    # from the MXFP8 oracle projects onto d with coefficient ~1 (~0 if x were quantised);
    # the bf16 rounding of y is uncorrelated with d
    y8 = run_oracle(wl)[key]
    d = ref[key] - y8
    c = float(np.vdot(g["y"] - y8, d) / np.vdot(d, d))
    _, f8 = errors(g["y"], y8)
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


CASES = [
    # T, K, N, fmt, ranks, seed
    (16, 4096, 28672, "fp8", [16] * 32, 41),              # gate-up shape, 16 tokens
    (16, 21504, 5376, "mxfp4", [8, 16, 32, 64] * 4, 42),  # MXFP4 down-projection shape
    (1, 128, 64, "fp8", [8], 43),
    (5, 256, 128, "mxfp4", [16, 8], 44),
    (13, 1152, 320, "fp8", [8, 24, 64], 45),
    (16, 640, 192, "mxfp4", [32, 16], 46),
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


def test_bf16_activations_token_limit():
    import torch
    import precision_gemm_amd as P
    from precision_gemm_amd._lib import LoraError
    from workloads.device import upload
    print("[case] act_bf16 T=17 rejected", flush=True)
    wl = workloads.make_custom(17, 256, 128, "fp8", [8], np.zeros(17, int), [1.0], 47)
    x, w, ad, ids = upload(wl)
    ws = P.alloc_workspace(wl.T, wl.K, wl.N, ad.n, ad.r_max)
    seg = P.build_segments(ids, ad.n)
    y = torch.full((17, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(LoraError) as ei:
        P.gemm_lowp_lora_epilogue(x, w, seg, ad, ws, y=y, act_bf16=True)
    assert ei.value.status == 2                  # LORA_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert (y == 3.0).all()                      # nothing was enqueued
