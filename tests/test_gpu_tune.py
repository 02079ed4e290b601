"""The down-projection's configurations on the GPU: every compiled configuration that the
search may visit gives t bitwise equal to lora_shrink's (the summation order does not depend
on the tiling, caching or scheduling), which is within the oracle's bound; a short search
returns a feasible configuration no slower than where it started."""

import numpy as np
import pytest

import workloads
from gpu_util import assert_t_close, run_oracle

pytestmark = pytest.mark.gpu

CASES = [  # T, K, ranks, ids: a single adapter, Zipf ids, one token per adapter, long segments
    (16, 2048, [16], "same"),
    (64, 1024, [16] * 12, "random"),
    (128, 1024, [8, 16, 32, 64] * 16, "distinct"),
    (300, 768, [64, 4, 20, 33], "sorted"),
]


@pytest.mark.parametrize("case", CASES, ids=[f"T{c[0]}_{c[3]}" for c in CASES])
def test_every_configuration_gives_the_same_t(case):
    import torch
    import precision_gemm_amd as P
    from precision_gemm_amd import tune
    from workloads.device import upload
    T, K, ranks, kind = case
    print(f"[case] shrink configurations {case}", flush=True)
    rng = np.random.default_rng(T)
    n = len(ranks)
    ids = {"same": np.zeros(T, int), "random": rng.integers(0, n, T),
           "distinct": rng.permutation(np.arange(T) % n), "sorted": np.sort(rng.integers(0, n, T))}[kind]
    wl = workloads.make_custom(T, K, 256, "fp8", ranks, ids, [1.0] * n, 800 + T, a_std=0.1)
    x, w, ad, idt = upload(wl)
    seg = P.build_segments(idt, ad.n)
    ref_t = P.shrink(x, seg, ad, None)
    torch.cuda.synchronize()
    assert_t_close(ref_t.cpu().numpy().astype(np.float64), run_oracle(wl)["t"], str(case))
    checked = 0
    for node in tune.space():
        tg, jp, u, m, order = node
        info = P.shrink_config_info(tg, jp, u)
        if not tune.feasible(node, lambda *a: info, T):
            continue
        t = torch.full_like(ref_t, -3.0)
        P.shrink_configured(x, seg, ad, tune.to_config(node), t=t)
        torch.cuda.synchronize()
        assert torch.equal(t, ref_t), (case, node)
        checked += 1
    print(f"  {checked} configurations bitwise equal", flush=True)
    assert checked >= 20


def test_short_search():
    import torch
    import precision_gemm_amd as P
    from precision_gemm_amd import tune
    from workloads.device import upload
    print("[case] short configuration search", flush=True)
    rng = np.random.default_rng(5)
    wl = workloads.make_custom(128, 2048, 256, "fp8", [8, 16, 32, 64] * 8, rng.permutation(np.arange(128) % 32),
                               [1.0] * 32, 805, a_std=0.1)
    x, w, ad, idt = upload(wl)
    seg = P.build_segments(idt, ad.n)
    res = tune.tune_shrink(x, seg, ad, steps=6, reps=3, seed=1)
    assert res.best_cost <= res.start_cost and len(res.trace) >= 1
    info = P.shrink_config_info(*res.best[:3])
    assert info["spill"] == 0
    t = P.shrink_configured(x, seg, ad, tune.to_config(res.best))
    ref = P.shrink(x, seg, ad, None)
    torch.cuda.synchronize()
    assert torch.equal(t, ref)
