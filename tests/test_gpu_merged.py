"""The per-token merged-weight formulation (lora_merged_layer, the alternative the "LoRA-Switch"
abstract describes) against the oracle.  By the merged-weight identity
x.(W_d + s_a A_a B_a) = x.W_d + s_a (x.A_a).B_a it equals the oracle's 16-bit-activation layer;
checked to the layer's bounds on single-adapter, many-adapter and mixed-rank batches in both
weight formats, with invalid adapter ids and ranks (base term only)."""

import numpy as np
import pytest

import workloads
from gpu_util import assert_y_close, bf16_to_f64, run_oracle

pytestmark = pytest.mark.gpu

CASES = [
    # T, K, N, fmt, ranks, ids
    (4, 256, 256, "fp8", [8, 8], [0, 1, 1, 0]),
    (16, 2048, 384, "fp8", [16], "zeros"),
    (16, 1024, 256, "mxfp4", [8, 16, 16, 32, 64, 8, 16, 32], "random"),
    (40, 1024, 320, "fp8", [1, 4, 12, 20, 60], "random"),
    (100, 512, 192, "mxfp4", [1, 3, 5], "random"),
    (7, 640, 64, "fp8", [64, 2], "random"),
]


def _ids(spec, T, n, rng):
    if isinstance(spec, list):
        return np.asarray(spec)
    return np.zeros(T, int) if spec == "zeros" else rng.integers(0, n, T)


@pytest.mark.parametrize("case", CASES, ids=[f"T{c[0]}_K{c[1]}_N{c[2]}_{c[3]}_a{len(c[4])}" for c in CASES])
def test_merged_layer_matches_oracle(case):
    import torch
    import precision_gemm_amd as P
    from workloads.device import upload
    T, K, N, fmt, ranks, spec = case
    print(f"[case] merged layer {case}", flush=True)
    rng = np.random.default_rng(T + K)
    ids = _ids(spec, T, len(ranks), rng)
    wl = workloads.make_custom(T, K, N, fmt, ranks, ids, [1.0 + 0.5 * i for i in range(len(ranks))], 900 + T,
                               a_std=0.1, b_std=0.05)
    x, w, ad, idt = upload(wl)
    wr = P.LowpWeight(fmt, torch.from_numpy(np.ascontiguousarray(wl.w_q)).cuda(),
                      torch.from_numpy(np.ascontiguousarray(wl.w_scale)).cuda())
    rows, ptrs = P.adapter_rows(ad)
    y = P.merged_layer(x, wr, idt, ad, ptrs)
    torch.cuda.synchronize()
    ref = run_oracle(wl, act="bf16")
    m, f = assert_y_close(bf16_to_f64(y), ref["y"], str(case))
    lora = np.linalg.norm(bf16_to_f64(y) - ref["y_base"] - ref["y_lora"]) / np.linalg.norm(ref["y_lora"])
    assert lora < 0.05, lora
    print(f"  y max_rel={m:.2e} frob={f:.2e} lora term rel={lora:.2e}", flush=True)


def test_merged_layer_invalid_ids_and_ranks_get_the_base_term():
    import torch
    import precision_gemm_amd as P
    from workloads.device import upload
    from oracle.layer import LowpWeight as OW, base_gemm_bf16
    print("[case] merged layer with invalid ids and ranks", flush=True)
    ids = np.array([0, 1, 2, 5, 1, -1, 0, 2, 2, 1, 0, 3], np.int32)
    T = ids.size
    ok = np.where((ids >= 0) & (ids < 3), ids, 0)
    wl = workloads.make_custom(T, 512, 128, "fp8", [16, 8, 24], ok, [1.0, 2.0, 0.5], 950, a_std=0.1, b_std=0.05)
    x, w, ad, _ = upload(wl)
    ad.ranks[2] = 0                                     # adapter 2 made invalid
    wr = P.LowpWeight("fp8", torch.from_numpy(wl.w_q).cuda(), torch.from_numpy(wl.w_scale).cuda())
    rows, ptrs = P.adapter_rows(ad)
    y = bf16_to_f64(P.merged_layer(x, wr, torch.from_numpy(ids).cuda(), ad, ptrs))
    good = np.flatnonzero((ids >= 0) & (ids < 2))
    base = np.flatnonzero(~((ids >= 0) & (ids < 2)))
    assert_y_close(y[good], run_oracle(wl, rows=tuple(good.tolist()), act="bf16")["y"], "valid")
    assert_y_close(y[base], base_gemm_bf16(wl.x[base], OW("fp8", wl.w_q, wl.w_scale)), "base only")
